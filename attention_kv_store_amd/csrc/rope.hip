// kv_store_rope_paged: the "RoPE + KV cache store" step in one pass.
//
// A layer's step list puts a rotary position embedding of Q and K right before
// attention and fuses it with the KV-cache write (Transformer 추론 커널 (3/10),
// §1-§2); the fused pass reads each new K row once, rotates it and writes it
// into its pool slot, copies V, and rotates Q in place, saving the round trip
// of a separate RoPE kernel (same page, §8).  The rotation is RoFormer's (Su
// et al. 2021, section 3.2): pair i of a token at position p turns by
// a = (p / pos_scale) * base^(-2 i / rotary_dim); pairs are (i, i + rd/2) or
// (2i, 2i + 1).
//
// One workgroup per token row.  Its angles depend on the token only, so they
// are formed once -- in double precision, which keeps a large p * theta exact
// to far below fp32 resolution before the reduction inside sincos -- and
// shared through LDS by every head.  A unit of work is two 16-byte chunks that
// hold EPC whole pairs (the j-th chunk of each half for neox; two adjacent
// chunks for interleaved), so every pair is rotated by one lane from
// registers; dims past rotary_dim and V are 16-byte copies.  HBM-bound: it
// moves each byte once.
#include <cmath>
#include <type_traits>

#include "kvs_device.hpp"
#include "kvs_internal.hpp"

namespace kvs {

template <bool BF16>
struct RopeIO {
  using E = typename std::conditional<BF16, uint16_t, float>::type;
  static constexpr int EPC = BF16 ? 8 : 4;   // elements per 16-byte chunk
  // chunk -> EPC floats
  __device__ __forceinline__ static void unpack(const u32x4& w, float* f) {
    if constexpr (BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16lo_to_f32(w[i]);
        f[2 * i + 1] = bf16hi_to_f32(w[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
    }
  }
  // EPC floats -> chunk (round to nearest even for bf16)
  __device__ __forceinline__ static u32x4 pack(const float* f) {
    u32x4 w;
    if constexpr (BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(f[i]);
    }
    return w;
  }
};

template <bool BF16>
__global__ __launch_bounds__(256) void rope_store_kernel(RopeParams p) {
  using IO = RopeIO<BF16>;
  using E = typename IO::E;
  constexpr int EPC = IO::EPC;
  __shared__ float s_cos[kRopeMaxPairs], s_sin[kRopeMaxPairs];

  const int64_t t = blockIdx.x;
  const int half = p.rd / 2;
  const int32_t pos = p.pos[t];
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    double sn, cs;
    sincos((double)pos * p.inv_scale * p.inv_freq[i], &sn, &cs);
    s_cos[i] = (float)cs;
    s_sin[i] = (float)sn;
  }
  __syncthreads();

  const int32_t slot = p.slots ? p.slots[t] : -1;
  const bool store = slot >= 0 && (int64_t)slot < p.num_slots;
  const int cpr = p.D / EPC;             // chunks per head row
  const int nu = p.rd / (2 * EPC);       // rotation units per head (two chunks each)
  const int ntail = cpr - 2 * nu;        // chunks past rotary_dim
  const int64_t kv_row = (int64_t)p.Hkv * p.D;   // elements per token row of K / V
  E* qrow = p.q ? static_cast<E*>(p.q) + t * (int64_t)p.Hq * p.D : nullptr;
  const E* krow = static_cast<const E*>(p.k_new) + t * kv_row;
  const E* vrow = static_cast<const E*>(p.v_new) + t * kv_row;
  E* kdst = static_cast<E*>(p.k_cache) + (int64_t)slot * kv_row;
  E* vdst = static_cast<E*>(p.v_cache) + (int64_t)slot * kv_row;

  // work: [Q rotation units][K rotation units][K tail chunks][V chunks]
  const int nq = qrow ? p.Hq * nu : 0;
  const int nk = store ? p.Hkv * nu : 0;
  const int nkt = store ? p.Hkv * ntail : 0;
  const int nv = store ? p.Hkv * cpr : 0;
  const int total = nq + nk + nkt + nv;
  for (int u = threadIdx.x; u < total; u += blockDim.x) {
    if (u < nq + nk) {
      // one rotation unit: head h, unit j
      const bool isq = u < nq;
      const int r = isq ? u : u - nq;
      const int h = r / nu, j = r - h * nu;
      // element offsets of the two chunks and the first pair index of each
      int da, db, ia, ib;
      if (p.style == 0) {   // neox: chunk j of each half; element e of both is pair j*EPC + e
        da = j * EPC;
        db = half + j * EPC;
        ia = ib = j * EPC;
      } else {              // interleaved: chunks 2j, 2j+1; elements (2m, 2m+1) are one pair
        da = 2 * j * EPC;
        db = da + EPC;
        ia = j * EPC;
        ib = j * EPC + EPC / 2;
      }
      const E* src = isq ? qrow + (int64_t)h * p.D : krow + (int64_t)h * p.D;
      float a[EPC], b[EPC];
      IO::unpack(ld16(src + da), a);
      IO::unpack(ld16(src + db), b);
      if (p.style == 0) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          const float c = s_cos[ia + e], s = s_sin[ia + e];
          const float x1 = a[e], x2 = b[e];
          a[e] = fmaf(x1, c, -x2 * s);
          b[e] = fmaf(x2, c, x1 * s);
        }
      } else {
#pragma unroll
        for (int m = 0; m < EPC / 2; ++m) {
          const float ca = s_cos[ia + m], sna = s_sin[ia + m];
          const float x1 = a[2 * m], x2 = a[2 * m + 1];
          a[2 * m] = fmaf(x1, ca, -x2 * sna);
          a[2 * m + 1] = fmaf(x2, ca, x1 * sna);
          const float cb = s_cos[ib + m], snb = s_sin[ib + m];
          const float y1 = b[2 * m], y2 = b[2 * m + 1];
          b[2 * m] = fmaf(y1, cb, -y2 * snb);
          b[2 * m + 1] = fmaf(y2, cb, y1 * snb);
        }
      }
      E* dst = isq ? qrow + (int64_t)h * p.D : kdst + (int64_t)h * p.D;
      st16(dst + da, IO::pack(a));
      st16(dst + db, IO::pack(b));
    } else if (u < nq + nk + nkt) {
      // K dims past rotary_dim: copied
      const int r = u - nq - nk;
      const int h = r / ntail, c = 2 * nu + (r - h * ntail);
      st16(kdst + (int64_t)h * p.D + c * EPC, ld16(krow + (int64_t)h * p.D + c * EPC));
    } else {
      // V: copied (row-contiguous over heads)
      const int c = u - nq - nk - nkt;
      st16(vdst + (int64_t)c * EPC, ld16(vrow + (int64_t)c * EPC));
    }
  }
}

hipError_t launch_rope_store(const RopeParams& p, DType dt, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  if (dt == DType::BF16)
    hipLaunchKernelGGL(rope_store_kernel<true>, dim3((unsigned)p.T), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(rope_store_kernel<false>, dim3((unsigned)p.T), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace kvs
