// Controls of the fake HIP runtime in fake_hip.cpp (test infrastructure).
#pragma once
#include <hip/hip_runtime_api.h>

void fake_set_arch(int dev, const char* arch);   // gcnArchName reported for a device
void fake_set_current(int dev);                  // the current device (null stream)
void fake_set_fail(int fail);                    // every runtime call fails
hipStream_t fake_stream(int dev);                // a stream handle on a device
long fake_count(const char* what);               // "sync", "d2h", "d2d", "prop"
