// The dQ kernel (attn_bwd_dq.hpp) at head dimension 256.
//
// At d = 256 a wave holds 32 query rows of Q and dO (128 registers) and a
// 32 x 256 fp32 dQ accumulator (128 registers), so the kernel runs one wave
// per SIMD with part of its state in the accumulation registers. This
// translation unit is compiled without the flag that places MFMA results in
// VGPRs (used everywhere else): with it, the compiler kept Q and dO in the
// accumulation registers and copied four of them back to VGPRs before every
// MFMA; without it they stay in VGPRs and the accumulator in the accumulation
// registers.
#include <type_traits>

#include "attn_bwd_dq.hpp"

namespace attn {

namespace {

template <typename E, int MASK, bool DROPOUT, bool OUT_F32>
hipError_t launch_one(const BwdArgs& a, hipStream_t stream) {
  const int nqb = (a.N + 127) / 128;
  const int tq = a.B * a.H * nqb;
  hipLaunchKernelGGL((attn_bwd_dq_kernel<E, 256, MASK, DROPOUT, OUT_F32>),
                     dim3(((tq + 7) / 8) * 8), dim3(kBwdThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename E, int MASK>
hipError_t launch_m(bool dropout, bool out_f32, const BwdArgs& a, hipStream_t s) {
  if (dropout) return out_f32 ? launch_one<E, MASK, true, true>(a, s)
                              : launch_one<E, MASK, true, false>(a, s);
  return out_f32 ? launch_one<E, MASK, false, true>(a, s)
                 : launch_one<E, MASK, false, false>(a, s);
}

template <typename E>
hipError_t launch_e(int mask, bool dropout, bool out_f32, const BwdArgs& a, hipStream_t s) {
  if (mask == kMaskCausal) return launch_m<E, kMaskCausal>(dropout, out_f32, a, s);
  if (mask == kMaskBand) return launch_m<E, kMaskBand>(dropout, out_f32, a, s);
  return launch_m<E, kMaskNone>(dropout, out_f32, a, s);
}

}  // namespace

hipError_t launch_bwd_dq256(int dtype, int mask, bool dropout, bool out_f32, const BwdArgs& a,
                            hipStream_t stream) {
  if (dtype == 1) return launch_e<Elem<bf16_t>>(mask, dropout, out_f32, a, stream);
  return launch_e<Elem<f16_t>>(mask, dropout, out_f32, a, stream);
}

}  // namespace attn
