// Arguments of the ring backward, passed from the C ABI to the kernels' host side.
#pragma once

#include "bwa.h"

namespace bwa {

struct BwdArgs {
  const bwa_tensor *q, *k, *v, *o, *dout, *dq, *dk, *dv;
  const float* lse;
  int n, sched, mode, causal;
  float scale;
  void* workspace;
};

}  // namespace bwa
