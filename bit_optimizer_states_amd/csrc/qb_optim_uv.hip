// qb_optim_uv.hip -- the fused 8-bit optimizer steps whose never-negative
// state (v of AdamW, Adam and LAMB; the state of RMSprop) is held in the
// unsigned dynamic 8-bit code: the UV instantiations of qb_optim_kernels.h,
// compiled apart from the signed ones.
#include "qb_optim_kernels.h"

namespace qb {
namespace optim_dispatch {

hipError_t optim_kind_uv(int opt, int B, int gdt, const OptLaunch& a) { return optim_kind<true>(opt, B, gdt, a); }

}  // namespace optim_dispatch
}  // namespace qb
