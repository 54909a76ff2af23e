// ffn.hip -- launches of the expert-grouped SwiGLU GEMMs for bf16 and int4
// routed weights (other code widths: ffn_lowbit.hip; MXFP4: ffn_mx.hip) and
// the fp32 path.
#include "ffn_kernels.h"

namespace moe {

hipError_t launch_ffn_bf16(const FfnArgs& a, hipStream_t s) {
  const int sf = a.n_shared ? a.shared_fmt : MOE_BF16;
  if (a.routed_fmt == MOE_BF16 && sf == MOE_BF16) return launch_pair<MOE_BF16, MOE_BF16>(a, s);
  if (a.routed_fmt == MOE_BF16 && sf == MOE_I8_ROW) return launch_pair<MOE_BF16, MOE_I8_ROW>(a, s);
  if (a.routed_fmt == MOE_I4_G32 && sf == MOE_BF16) return launch_pair<MOE_I4_G32, MOE_BF16>(a, s);
  if (a.routed_fmt == MOE_I4_G32 && sf == MOE_I8_ROW)
    return launch_pair<MOE_I4_G32, MOE_I8_ROW>(a, s);
  if (ig32_bits(a.routed_fmt) != 0) return launch_ffn_lowbit(a, s);
  if (a.routed_fmt == MOE_MXFP4) return launch_ffn_mx(a, s);
  return hipErrorInvalidValue;
}

// ---- fp32 path: plain fp32 FMAs on canonical row-major weights --------------
// Block = one row tile x 64 columns, one thread per column, rows in sequence.
__global__ __launch_bounds__(64) void ffn_f32_stage1(FfnArgs A, int NB) {
  TileJob J;
  if (!decode_job(A, NB, A.F / 64, A.n_shared ? A.Fs / 64 : 0, BM, J)) return;
  const int Fw = J.shared ? A.Fs : A.F;
  const int j = J.nb * 64 + threadIdx.x;
  const float* blob = (const float*)(J.shared ? A.shared_blob
                                              : A.routed_blob + (size_t)J.expert * expert_bytes(MOE_F32, A.d, A.F));
  const float* wg = blob + (size_t)j * A.d;
  const float* wu = blob + (size_t)(Fw + j) * A.d;
  float* hout = (float*)(J.shared ? A.h_shared : A.h_routed);
  const float* X = (const float*)A.hidden;
  for (int m = 0; m < J.cnt; m++) {
    int t;
    float wf;
    if (J.shared) {
      t = J.start + m;
      wf = 1.0f;
    } else {
      const int f = A.perm[J.start + m];
      t = f / A.k;
      wf = A.topk_w[f];
    }
    const float* x = X + (size_t)t * A.d;
    float g = 0.0f, u = 0.0f;
    for (int i = 0; i < A.d; i++) {
      g = fmaf(wg[i], x[i], g);
      u = fmaf(wu[i], x[i], u);
    }
    hout[(size_t)(J.start + m) * Fw + j] = wf * (g / (1.0f + expf(-g))) * u;
  }
}

__global__ __launch_bounds__(64) void ffn_f32_stage2(FfnArgs A, int NB) {
  TileJob J;
  if (!decode_job(A, NB, NB, NB, BM, J)) return;
  const int Fw = J.shared ? A.Fs : A.F;
  const int n = J.nb * 64 + threadIdx.x;
  const float* blob = (const float*)(J.shared ? A.shared_blob
                                              : A.routed_blob + (size_t)J.expert * expert_bytes(MOE_F32, A.d, A.F));
  const float* wd = blob + (size_t)2 * Fw * A.d + (size_t)n * Fw;
  const float* H = (const float*)(J.shared ? A.h_shared : A.h_routed);
  float* out = J.shared ? A.shared_out : A.out_assign;
  for (int m = 0; m < J.cnt; m++) {
    const float* h = H + (size_t)(J.start + m) * Fw;
    float o = 0.0f;
    for (int j = 0; j < Fw; j++) o = fmaf(wd[j], h[j], o);
    out[(size_t)(J.start + m) * A.d + n] = o;
  }
}

hipError_t launch_ffn_f32(const FfnArgs& a0, hipStream_t s) {
  FfnArgs a = a0;
  a.shared_slots = a.n_shared ? (a.T + BM - 1) / BM : 0;
  const int slots = (a.routed_slots + a.shared_slots + 7) / 8 * 8;
  const int nb1 = max(a.F, a.n_shared ? a.Fs : 0) / 64, nb2 = a.d / 64;
  ffn_f32_stage1<<<slots * nb1, 64, 0, s>>>(a, nb1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  ffn_f32_stage2<<<slots * nb2, 64, 0, s>>>(a, nb2);
  return hipGetLastError();
}

}  // namespace moe
