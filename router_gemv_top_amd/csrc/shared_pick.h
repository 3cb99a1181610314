// shared_pick.h - the router + shared-expert SwiGLU kernel's instances
// (built in shared_inst.hip). Returns the kernel for the router tile of the
// plan: VALU tile of mt rows (1, 2, 4, 8) with l 512-element k-chunks per
// lane (1, 2, 4, 7), or the 16-row MFMA tile (mt 1) with ks 32-element
// k-steps per wave (2, 4, 8), whose shared part is the VALU form of 8 rows
// for m <= 8 and the MFMA form above; nullptr for any other shape. Kernel
// arguments: (GemvArgs, SharedArgs, int router_workgroups).
#pragma once

namespace rgt {

const void* shared_pick(bool valu, int mt, int l, int ks, int m);

}  // namespace rgt
