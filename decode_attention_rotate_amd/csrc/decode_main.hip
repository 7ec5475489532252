// Decode and prefill attention: split combination and the tables of split-K
// kernel instantiations.
//
// Combination merges the per-split (max, sum, weighted V) triples with the
// log-sum-exp rule and rotates the result back to the original space
// (velog.io post "fix KV cache quantization outliers", section "Hadamard
// rotation": the attention result is inverse-rotated).
#include "common.hpp"
#include "kernels.hpp"

namespace kvq {

// Tables defined by the instantiation units, indexed [V format][G-1] with V
// formats q4_0, q5_0, q6_0, q8_0, q4_1, q5_1; one pair of tables per (D, K
// width, K block kind).
#define KVQ_DECLARE_TABLE(D, KB, KM) extern DecodeLauncher kvq_decode_table_##D##_##KB##_##KM[6][8]; \
  extern DecodeLauncher kvq_prefill_table_##D##_##KB##_##KM[6];
#define KVQ_ALL_K(X, D) X(D, 4, 0) X(D, 5, 0) X(D, 6, 0) X(D, 8, 0) X(D, 4, 1) X(D, 5, 1)
KVQ_ALL_K(KVQ_DECLARE_TABLE, 64) KVQ_ALL_K(KVQ_DECLARE_TABLE, 128)
KVQ_ALL_K(KVQ_DECLARE_TABLE, 192) KVQ_ALL_K(KVQ_DECLARE_TABLE, 256)
#define KVQ_DECLARE_PTABLE(D, KB, KM) extern DecodeLauncher kvq_decode_ptable_##D##_##KB##_##KM[6][8]; \
  extern DecodeLauncher kvq_prefill_ptable_##D##_##KB##_##KM[6];
KVQ_ALL_K(KVQ_DECLARE_PTABLE, 256)
// outlier-channel kernels: head_dim 128, absmax K, [V format q4_0..q8_0][G-1]
#define KVQ_DECLARE_OTABLE(D, KB, KM) extern DecodeLauncher kvq_decode_otable_##D##_##KB##_##KM[4][8];
KVQ_DECLARE_OTABLE(128, 4, 0) KVQ_DECLARE_OTABLE(128, 5, 0) KVQ_DECLARE_OTABLE(128, 6, 0)
KVQ_DECLARE_OTABLE(128, 8, 0)
#undef KVQ_DECLARE_TABLE

namespace {
int v_index(int vb, bool vm) {
  if (vm) return vb == 4 ? 4 : vb == 5 ? 5 : -1;
  return vb == 4 ? 0 : vb == 5 ? 1 : vb == 6 ? 2 : vb == 8 ? 3 : -1;
}
}  // namespace

DecodeLauncher decode_launcher(int D, int kb, int vb, int gc, bool km, bool vm, bool paged,
                               bool outliers) {
  const int vi = v_index(vb, vm);
  if (vi < 0 || gc < 1 || gc > 8) return nullptr;
  if (outliers) {
    if (D != 128 || km || vm || vi > 3) return nullptr;
    if (kb == 4) return kvq_decode_otable_128_4_0[vi][gc - 1];
    if (kb == 5) return kvq_decode_otable_128_5_0[vi][gc - 1];
    if (kb == 6) return kvq_decode_otable_128_6_0[vi][gc - 1];
    if (kb == 8) return kvq_decode_otable_128_8_0[vi][gc - 1];
    return nullptr;
  }
  if (paged && split_fixed_layout(D)) {
#define KVQ_PICK(DD, KK, MM) \
  if (D == DD && kb == KK && (int)km == MM) return kvq_decode_ptable_##DD##_##KK##_##MM[vi][gc - 1];
    KVQ_ALL_K(KVQ_PICK, 256)
#undef KVQ_PICK
    return nullptr;
  }
#define KVQ_PICK(DD, KK, MM) \
  if (D == DD && kb == KK && (int)km == MM) return kvq_decode_table_##DD##_##KK##_##MM[vi][gc - 1];
  KVQ_ALL_K(KVQ_PICK, 64) KVQ_ALL_K(KVQ_PICK, 128) KVQ_ALL_K(KVQ_PICK, 192) KVQ_ALL_K(KVQ_PICK, 256)
#undef KVQ_PICK
  return nullptr;
}

DecodeLauncher prefill_launcher(int D, int kb, int vb, bool km, bool vm, bool paged) {
  const int vi = v_index(vb, vm);
  if (vi < 0) return nullptr;
  if (paged && split_fixed_layout(D)) {
#define KVQ_PICK(DD, KK, MM) \
  if (D == DD && kb == KK && (int)km == MM) return kvq_prefill_ptable_##DD##_##KK##_##MM[vi];
    KVQ_ALL_K(KVQ_PICK, 256)
#undef KVQ_PICK
    return nullptr;
  }
#define KVQ_PICK(DD, KK, MM) \
  if (D == DD && kb == KK && (int)km == MM) return kvq_prefill_table_##DD##_##KK##_##MM[vi];
  KVQ_ALL_K(KVQ_PICK, 64) KVQ_ALL_K(KVQ_PICK, 128) KVQ_ALL_K(KVQ_PICK, 192) KVQ_ALL_K(KVQ_PICK, 256)
#undef KVQ_PICK
  return nullptr;
}
#undef KVQ_ALL_K

namespace {

// Block-wide reductions of a 256-thread block (4 waves).
__device__ inline float block_max(float v, float* red) {
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
  const int t = threadIdx.x;
  __syncthreads();
  if ((t & 63) == 0) red[t >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}
__device__ inline float block_sum(float v, float* red) {
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m);
  const int t = threadIdx.x;
  __syncthreads();
  if ((t & 63) == 0) red[t >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// One 256-thread block per (sequence, query head), log-sum-exp merge of the
// S split partials: M = max m_s, w_s = 2^(m_s - M), out = sum w_s acc_s /
// sum w_s l_s, then the inverse rotation.  The weights go to LDS once;
// thread t < P * D then sums element t % D over the splits s = t / D (mod
// P = 256 / D; at head_dim 192 the last 64 threads sum nothing) with several
// loads in flight.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  constexpr int P = 256 / D;       // split phases handled in parallel
  constexpr int U = 4;             // independent partial sums per thread
  __shared__ float wgt[kMaxSplitsDevice];
  __shared__ float red[256];
  __shared__ float o[D];
  const int t = threadIdx.x;
  const int bh = blockIdx.x;
  const int S = a.S;
  const float* ml = a.part_ml + (size_t)bh * S * 2;
  const float* acc = a.part_acc + (size_t)bh * S * D;
  float mloc = -INFINITY;
  for (int s = t; s < S; s += 256) mloc = fmaxf(mloc, ml[2 * s]);
  const float M = block_max(mloc, red);
  float lsum = 0.f;
  for (int s = t; s < S; s += 256) {
    const float m = ml[2 * s];
    const float w = m == -INFINITY ? 0.f : exp2f(m - M);
    wgt[s] = w;
    lsum += w * ml[2 * s + 1];
  }
  const float L = block_sum(lsum, red);   // its barriers also publish wgt
  // outlier channels of V: thread t < 32 merges channel slot t the same way
  float vo = 0.f;
  if (a.part_out && t < kOutl) {
    const float* po = a.part_out + (size_t)bh * S * kOutl + t;
    for (int s2 = 0; s2 < S; ++s2) vo += wgt[s2] * po[(size_t)s2 * kOutl];
  }
  const int e = t % D, ph = t / D;
  float v[U] = {};
  int s = t < P * D ? ph : S;
  for (; s + (U - 1) * P < S; s += U * P) {
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] += wgt[s + u * P] * acc[(size_t)(s + u * P) * D + e];
  }
  for (; s < S; s += P) v[0] += wgt[s] * acc[(size_t)s * D + e];
  __syncthreads();                        // every thread has read red[0..3]
  red[t] = (v[0] + v[1]) + (v[2] + v[3]);
  __syncthreads();
  if (t < D) {
    float tot = 0.f;
#pragma unroll
    for (int k = 0; k < P; ++k) tot += red[t + k * D];
    o[t] = tot;
  }
  __syncthreads();
  if (a.rotate) {
    for (int h = 1; h < rot_block(D); h <<= 1) {   // head_dim 192: within each H_64 block
      if (t < D / 2) {
        const int i = (t / h) * 2 * h + (t % h);
        const float u = o[i], w = o[i + h];
        o[i] = u + w;
        o[i + h] = u - w;
      }
      __syncthreads();
    }
  }
  const float scale = (a.rotate ? a.cd : 1.0f) / L;
  float r = 0.f;
  if (t < D) {
    r = o[t] * scale;
    if (a.rotate && a.has_signs)   // back by diag(s) H
      r = __uint_as_float(__float_as_uint(r) ^ (((a.signs[t / 32] >> (t % 32)) & 1u) << 31));
  }
  if (a.part_out) {
    // the outlier channels' part is added at V's channels (original space)
    __syncthreads();   // every thread has read o[] for the rotation
    if (t < D) o[t] = r;
    __syncthreads();
    if (t < kOutl) {
      const int g = (bh % a.Hq) / a.G;
      const int ch = outlier_channel(a.v_out_idx + (size_t)g * kOutl, t, D);
      o[ch] = o[ch] + vo / L;   // the channels of a list are distinct
    }
    __syncthreads();
    if (t < D) r = o[t];
  }
  if (t < D) a.out[(size_t)bh * D + t] = r;
}

}  // namespace

hipError_t launch_combine(int D, const CombineArgs& a, int B, hipStream_t s) {
  (void)hipGetLastError();  // drop errors left by earlier runtime calls
  const dim3 grid(B * a.Hq);
  switch (D) {
    case 64: hipLaunchKernelGGL(combine_kernel<64>, grid, dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL(combine_kernel<128>, grid, dim3(256), 0, s, a); break;
    case 192: hipLaunchKernelGGL(combine_kernel<192>, grid, dim3(256), 0, s, a); break;
    case 256: hipLaunchKernelGGL(combine_kernel<256>, grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvq
