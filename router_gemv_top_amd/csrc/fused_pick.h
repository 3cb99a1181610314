// fused_pick.h - the fused kernel's instances, one translation unit per
// expert-count bucket and norm flag (fused_inst.hip built with RGT_NV = 2, 4,
// 8, 14, 16: lanes hold up to NV*64 experts; RGT_NORM = 0, 1), so the
// instances compile in parallel. Each returns the kernel for a tile kind and
// shape, for hipLaunchKernel.
#pragma once

namespace rgt {

// valu: VALU tile of mt rows (1, 2, 4, 8) with l 512-element k-chunks per
// lane (1, 2, 4, 7); otherwise MFMA tile of mt 16-row tiles (1..4) with ks
// 32-element k-steps per wave (2, 4, 8).
const void* fused_pick_nv2(bool valu, int mt, int l, int ks);
const void* fused_pick_nv4(bool valu, int mt, int l, int ks);
const void* fused_pick_nv8(bool valu, int mt, int l, int ks);
const void* fused_pick_nv14(bool valu, int mt, int l, int ks);
const void* fused_pick_nv16(bool valu, int mt, int l, int ks);

// The same instances behind the RMSNorm producer (the tile and the quant
// read the norm of x; FusedArgs' norm fields set).
const void* fused_norm_pick_nv2(bool valu, int mt, int l, int ks);
const void* fused_norm_pick_nv4(bool valu, int mt, int l, int ks);
const void* fused_norm_pick_nv8(bool valu, int mt, int l, int ks);
const void* fused_norm_pick_nv14(bool valu, int mt, int l, int ks);
const void* fused_norm_pick_nv16(bool valu, int mt, int l, int ks);

}  // namespace rgt
