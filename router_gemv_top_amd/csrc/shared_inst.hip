// shared_inst.hip - instances of the router + shared-expert SwiGLU kernel
// (one translation unit of its own, so they compile beside the others).
#include <hip/hip_runtime.h>

#include "shared.h"
#include "shared_pick.h"

namespace rgt {

template <int MT>
static const void* pick_valu(int l) {
  switch (l) {
    case 1: return reinterpret_cast<const void*>(&router_shared_kernel<MT, 1, 0>);
    case 2: return reinterpret_cast<const void*>(&router_shared_kernel<MT, 2, 0>);
    case 4: return reinterpret_cast<const void*>(&router_shared_kernel<MT, 4, 0>);
    case 7: return reinterpret_cast<const void*>(&router_shared_kernel<MT, 7, 0>);
    default: return nullptr;
  }
}

const void* shared_pick(bool valu, int mt, int l, int ks, int m) {
  if (valu) {
    switch (mt) {
      case 1: return pick_valu<1>(l);
      case 2: return pick_valu<2>(l);
      case 4: return pick_valu<4>(l);
      case 8: return pick_valu<8>(l);
      default: return nullptr;
    }
  }
  if (mt != 1) return nullptr;
  if (m <= 8) {  // the shared part's VALU form for up to 8 rows
    switch (ks) {
      case 2: return reinterpret_cast<const void*>(&router_shared_kernel<1, 1, 2, 8>);
      case 4: return reinterpret_cast<const void*>(&router_shared_kernel<1, 1, 4, 8>);
      case 8: return reinterpret_cast<const void*>(&router_shared_kernel<1, 1, 8, 8>);
      default: return nullptr;
    }
  }
  switch (ks) {
    case 2: return reinterpret_cast<const void*>(&router_shared_kernel<1, 1, 2>);
    case 4: return reinterpret_cast<const void*>(&router_shared_kernel<1, 1, 4>);
    case 8: return reinterpret_cast<const void*>(&router_shared_kernel<1, 1, 8>);
    default: return nullptr;
  }
}

}  // namespace rgt
