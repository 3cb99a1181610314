// fused_inst.hip - instances of the one-launch decode kernel for one
// expert-count bucket, chosen at build time by RGT_NV, with or without the
// RMSNorm producer in front (RGT_NORM; see fused_pick.h).
#include <hip/hip_runtime.h>

#include "fused.h"
#include "fused_pick.h"

#ifndef RGT_NV
#error "build with -DRGT_NV=<2|4|8|14|16>"
#endif
#ifndef RGT_NORM
#error "build with -DRGT_NORM=<0|1>"
#endif

#define RGT_CAT2(a, b) a##b
#define RGT_CAT(a, b) RGT_CAT2(a, b)
#if RGT_NORM
#define RGT_PICK RGT_CAT(fused_norm_pick_nv, RGT_NV)
#else
#define RGT_PICK RGT_CAT(fused_pick_nv, RGT_NV)
#endif

namespace rgt {
namespace {

constexpr bool kNorm = RGT_NORM != 0;

template <int MT>
const void* valu_ptr(int l) {
  switch (l) {
    case 1: return (const void*)fused_valu_kernel<RGT_NV, kNorm, MT, 1, 1>;
    case 2: return (const void*)fused_valu_kernel<RGT_NV, kNorm, MT, 1, 2>;
    case 4: return (const void*)fused_valu_kernel<RGT_NV, kNorm, MT, 1, 4>;
    default: return (const void*)fused_valu_kernel<RGT_NV, kNorm, MT, 1, 7>;
  }
}

template <int MT>
const void* mfma_ptr(int ks) {
  switch (ks) {
    case 2: return (const void*)fused_mfma_kernel<RGT_NV, kNorm, MT, 2>;
    case 4: return (const void*)fused_mfma_kernel<RGT_NV, kNorm, MT, 4>;
    default: return (const void*)fused_mfma_kernel<RGT_NV, kNorm, MT, 8>;
  }
}

}  // namespace

const void* RGT_PICK(bool valu, int mt, int l, int ks) {
  if (valu) {
    switch (mt) {
      case 1: return valu_ptr<1>(l);
      case 2: return valu_ptr<2>(l);
      case 4: return valu_ptr<4>(l);
      default: return valu_ptr<8>(l);
    }
  }
  switch (mt) {
    case 1: return mfma_ptr<1>(ks);
    case 2: return mfma_ptr<2>(ks);
    case 3: return mfma_ptr<3>(ks);
    default: return mfma_ptr<4>(ks);
  }
}

}  // namespace rgt
