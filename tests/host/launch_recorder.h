// Launches recorded by launch_recorder.cpp (test infrastructure).
#pragma once
#include <vector>

#include "gg_kernels.h"

struct Launch {
    const char* kind;
    gg::GemmParams p;
    int num_cu;
    const uint16_t* packed;   // pack_frag
    uint16_t* frag;           // pack_frag
    int a, b, c;              // pack_frag: E, H, F; round_bf16: n; dp_reduce: E, M, ld;
                              // scale_rows(_bwd): M, H, dprobs != null
};
extern std::vector<Launch> g_launches;
