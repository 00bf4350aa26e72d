// Internal interface between the C-ABI entry points (fa_api.hip) and the
// kernel launchers (fa_fwd.hip, fa_bwd.hip).  Arguments arrive here already
// validated: non-null, 16-byte aligned, d in {64, 128}, N >= 1, B*H >= 1,
// finite non-negative scale.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

enum Dt { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

constexpr float kLog2eHost = 1.4426950408889634f;

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int BH;     // batch * heads
  int N;      // sequence length (queries = keys)
  int d;      // head dimension
  float c;    // scale * log2(e)
  int causal;
  int dtype;
  hipStream_t stream;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* dvec;  // workspace: D_i = dO_i . O_i, [B*H*N] fp32
  int BH;
  int N;
  int d;
  float scale;
  float c;      // scale * log2(e)
  int causal;
  int dtype;
  hipStream_t stream;
};

enum BwdStage { BWD_PREP = 0, BWD_DKDV = 1, BWD_DQ = 2 };

hipError_t launch_fwd(const FwdArgs& a);
hipError_t launch_bwd(const BwdArgs& a);                 // all three stages in order
hipError_t launch_bwd_stage(const BwdArgs& a, int stage);  // one stage

}  // namespace fa
