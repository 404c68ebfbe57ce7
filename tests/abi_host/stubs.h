// Counters and the last launch shape recorded by the host stand-ins.
#pragma once
#include "../../mxfp4_activation_amd/csrc/wush_kernels.h"

struct StubQuant {
  int fmt;  // -1 for the AbsMax pass
  wush::QuantArgs args;
  int n_wg;
};

extern int g_hip_calls;
extern int g_launches;
extern StubQuant g_last_quant;
