// Decode attention (one query row per sequence) over the paged KV cache.
//
// Decode scans a long paged K/V context per sequence with few query rows, so it
// is bound by HBM bandwidth and needs its own work split (Transformer 추론 커널
// (3/10), §13).  Long or uneven contexts are cut into key chunks whose partial
// results (m_i, l_i, O_i) are merged afterwards in a numerically stable way
// (same page, §16), using the running-statistics update of §12.
//
// Pass 1 (decode_split_kernel): one wave per (sequence, KV head, key chunk).
//  * The G query heads that share the KV head ride in the 16 columns of the
//    MFMA (G <= 16; unused columns are zero), so each K/V byte is read once
//    for the whole group (§15).
//  * S^T = K . Q^T with the 16x16x32 bf16 MFMA: the A operand (16 keys x 32 d)
//    is exactly one 16-byte global load per lane from the paged pool, so K
//    goes HBM -> registers with no LDS hop.
//  * The accumulator layout of S^T (lane: one query column, 4 keys) is the B
//    operand layout of the 16x16x16 MFMA, so P feeds O^T = V^T . P^T directly.
//    V is transposed through a small per-wave LDS slab (d-major rows of 16
//    keys, padded to 40 bytes so the 8-byte reads are bank-conflict free).
//  * The next step's K/V loads are issued before the current step's math
//    (two register buffers), and block-table entries are scalar loads.
//  * Writes the normalised partial O_i and its base-2 lse_i, or the final
//    out/lse directly when the sequence has a single chunk.
// Pass 2 (decode_merge_kernel): per (row, head, d): lse = M + log2 sum
//  exp2(lse_i - M), out = sum exp2(lse_i - lse) O_i.  Chunks past a sequence's
//  end are never written or read.
#include <type_traits>

#include "kvs_device.hpp"
#include "kvs_internal.hpp"

namespace kvs {

template <int D>
struct DCfg {
  static constexpr int NBS = D == 64 ? 4 : 2;     // 16-key blocks per step
  static constexpr int KEYS = NBS * 16;           // keys per step
  static constexpr int KI = D / 32;               // 16x16x32 k-steps over d
  static constexpr int NDB = D / 16;              // 16-wide d blocks of the output
  static constexpr int VROW = 40;                 // bytes per V^T row (16 keys + pad)
  static constexpr int VBLK = D * VROW;           // V^T bytes per 16-key block
  static constexpr int VITEMS = 8 * (D / 8);      // (key pair, 8-d chunk) items per block
  static constexpr int VIL = VITEMS / 64;         // items per lane per block
};

template <int D, bool BF16>
__global__ __launch_bounds__(64) void decode_split_kernel(AttnParams p) {
  using C = DCfg<D>;
  const int lane = threadIdx.x;
  const int col = lane & 15, grp = lane >> 4;
  const int sp = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int Lk = p.lens_k[b];
  // clamped so a max_seqlen_k hint below a real length stays in bounds
  const int nsplit = min((Lk + p.chunk - 1) / p.chunk, p.max_splits);
  if (sp >= nsplit) return;
  const int kbeg = sp * p.chunk;
  const int kend = min(Lk, kbeg + p.chunk);
  const int nsteps = (kend - kbeg + C::KEYS - 1) / C::KEYS;
  const int t = p.cu_q[b];
  const bool head_ok = col < p.G;
  const int h = g * p.G + (head_ok ? col : 0);
  const int32_t* trow = p.table + (int64_t)b * p.MB;
  const int64_t tok_stride = (int64_t)p.Hkv * D;

  using E = typename std::conditional<BF16, uint16_t, float>::type;
  const E* kbase = static_cast<const E*>(p.k) + (int64_t)g * D;
  const E* vbase = static_cast<const E*>(p.v) + (int64_t)g * D;
  const E* qp = static_cast<const E*>(p.q) + ((int64_t)t * p.Hq + h) * D;

  float m_run = kMaskedScore, l_run = 0.f;
  f32x4 o[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) o[db] = f32x4{};

  if constexpr (BF16) {
    __shared__ __attribute__((aligned(16))) char vt[C::NBS * C::VBLK];
    // B operand of S^T = K . Q^T: lane holds Q[col][i*32 + grp*8 .. +8]
    u32x4 qf[C::KI];
#pragma unroll
    for (int i = 0; i < C::KI; ++i) qf[i] = head_ok ? ld16(qp + i * 32 + grp * 8) : u32x4{0, 0, 0, 0};

    u32x4 kA[C::NBS][C::KI], kB[C::NBS][C::KI];
    u32x4 vA[C::NBS][2 * C::VIL], vB[C::NBS][2 * C::VIL];
    // K: lane reads row (lane % 16) of each block, d = i*32 + grp*8.
    // V: lane reads the two rows of key pair kp = lane % 8 at d-chunk
    //    lane / 8 (+ 8 per extra item).
    auto load = [&](int step, u32x4 (&kr)[C::NBS][C::KI], u32x4 (&vr)[C::NBS][2 * C::VIL]) {
      const int k0 = kbeg + step * C::KEYS;
#pragma unroll
      for (int j = 0; j < C::NBS; ++j) {
        const int kb0 = k0 + 16 * j;
        const bool blk_ok = kb0 < kend;
        const int phys = blk_ok ? trow[kb0 >> 4] : 0;
        const E* kblk = kbase + (int64_t)phys * kPage * tok_stride;
        const E* vblk = vbase + (int64_t)phys * kPage * tok_stride;
        const bool krow_ok = kb0 + col < kend;
#pragma unroll
        for (int i = 0; i < C::KI; ++i)
          kr[j][i] = krow_ok ? ld16(kblk + col * tok_stride + i * 32 + grp * 8) : u32x4{0, 0, 0, 0};
        const int kp = lane & 7;
        const bool v0_ok = kb0 + 2 * kp < kend, v1_ok = kb0 + 2 * kp + 1 < kend;
#pragma unroll
        for (int it = 0; it < C::VIL; ++it) {
          const int dch = (lane >> 3) + 8 * it;
          vr[j][2 * it] = v0_ok ? ld16(vblk + (2 * kp) * tok_stride + dch * 8) : u32x4{0, 0, 0, 0};
          vr[j][2 * it + 1] = v1_ok ? ld16(vblk + (2 * kp + 1) * tok_stride + dch * 8) : u32x4{0, 0, 0, 0};
        }
      }
    };
    auto compute = [&](int step, const u32x4 (&kr)[C::NBS][C::KI], const u32x4 (&vr)[C::NBS][2 * C::VIL]) {
      const int k0 = kbeg + step * C::KEYS;
      // V^T into LDS: word (V[2kp][d], V[2kp+1][d]) at row d, key pair kp
      __syncthreads();
#pragma unroll
      for (int j = 0; j < C::NBS; ++j) {
        const int kp = lane & 7;
#pragma unroll
        for (int it = 0; it < C::VIL; ++it) {
          const int dch = (lane >> 3) + 8 * it;
          const u32x4 w0 = vr[j][2 * it], w1 = vr[j][2 * it + 1];
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            char* r0 = vt + j * C::VBLK + (dch * 8 + 2 * m) * C::VROW + kp * 4;
            *reinterpret_cast<uint32_t*>(r0) = __builtin_amdgcn_perm(w1[m], w0[m], 0x05040100u);
            *reinterpret_cast<uint32_t*>(r0 + C::VROW) = __builtin_amdgcn_perm(w1[m], w0[m], 0x07060302u);
          }
        }
      }
      // scores
      f32x4 s[C::NBS];
#pragma unroll
      for (int j = 0; j < C::NBS; ++j) {
        s[j] = f32x4{};
#pragma unroll
        for (int i = 0; i < C::KI; ++i) s[j] = mfma16x16x32_bf16(kr[j][i], qf[i], s[j]);
      }
      float mt = kMaskedScore;
      const bool tail = k0 + C::KEYS > kend;
#pragma unroll
      for (int j = 0; j < C::NBS; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float x = s[j][r] * p.scale_log2;
          if (tail) x = (k0 + 16 * j + grp * 4 + r < kend) ? x : kMaskedScore;
          s[j][r] = x;
          mt = fmaxf(mt, x);
        }
      mt = fmaxf(mt, xor16(mt));
      mt = max_xor32(mt);
      const float m_new = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      float lsum = 0.f;
#pragma unroll
      for (int j = 0; j < C::NBS; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = __builtin_amdgcn_exp2f(s[j][r] - m_new);
          s[j][r] = e;
          lsum += e;
        }
      l_run = l_run * alpha + lsum;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) o[db] *= alpha;
      __syncthreads();
      // O^T += V^T . P^T
#pragma unroll
      for (int j = 0; j < C::NBS; ++j) {
        const u32x2 pb = {pack_bf16x2(s[j][0], s[j][1]), pack_bf16x2(s[j][2], s[j][3])};
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
          const u32x2 a = *reinterpret_cast<const u32x2*>(vt + j * C::VBLK + (db * 16 + col) * C::VROW + grp * 8);
          o[db] = mfma16x16x16_bf16(a, pb, o[db]);
        }
      }
    };

    load(0, kA, vA);
    for (int step = 0; step < nsteps; step += 2) {
      if (step + 1 < nsteps) load(step + 1, kB, vB);
      compute(step, kA, vA);
      if (step + 1 < nsteps) {
        if (step + 2 < nsteps) load(step + 2, kA, vA);
        compute(step + 1, kB, vB);
      }
    }
  } else {
    // fp32: 16x16x4 MFMA, one element per lane per operand; k-slot grp of
    // step i covers d = grp * D/4 + i.
    constexpr int QF = D / 4;
    float qf[QF];
#pragma unroll
    for (int c4 = 0; c4 < QF / 4; ++c4) {
      const u32x4 w = head_ok ? ld16(qp + grp * QF + c4 * 4) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 4; ++e) qf[c4 * 4 + e] = __uint_as_float(w[e]);
    }
    const int nblk = (kend - kbeg + 15) >> 4;
    for (int j = 0; j < nblk; ++j) {
      const int kb0 = kbeg + 16 * j;
      const int phys = trow[kb0 >> 4];
      const float* kblk = static_cast<const float*>(static_cast<const void*>(kbase)) + (int64_t)phys * kPage * tok_stride;
      const float* vblk = static_cast<const float*>(static_cast<const void*>(vbase)) + (int64_t)phys * kPage * tok_stride;
      f32x4 s = f32x4{};
      const bool krow_ok = kb0 + col < kend;
#pragma unroll
      for (int c4 = 0; c4 < QF / 4; ++c4) {
        const u32x4 w = krow_ok ? ld16(kblk + col * tok_stride + grp * QF + c4 * 4) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 4; ++e) s = mfma16x16x4_f32(__uint_as_float(w[e]), qf[c4 * 4 + e], s);
      }
      float mt = kMaskedScore;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = s[r] * p.scale_log2;
        x = (kb0 + grp * 4 + r < kend) ? x : kMaskedScore;
        s[r] = x;
        mt = fmaxf(mt, x);
      }
      mt = fmaxf(mt, xor16(mt));
      mt = max_xor32(mt);
      const float m_new = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      float lsum = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[r] = __builtin_amdgcn_exp2f(s[r] - m_new);
        lsum += s[r];
      }
      l_run = l_run * alpha + lsum;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) o[db] *= alpha;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = grp * 4 + r;
        const bool ok = kb0 + key < kend;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
          const float v = ok ? vblk[key * tok_stride + db * 16 + col] : 0.f;
          o[db] = mfma16x16x4_f32(v, s[r], o[db]);
        }
      }
    }
  }

  // ---- finish the chunk: combine the 4 lane groups' shares of l ----------
  float l_tot = l_run + xor16(l_run);
  l_tot = sum_xor32(l_tot);
  if (!head_ok) return;
  const float inv = 1.0f / l_tot;
  const float lse2 = m_run + __builtin_amdgcn_logf(l_tot);
  if (nsplit == 1) {
    const int64_t orow = ((int64_t)t * p.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      const int d = db * 16 + grp * 4;
      const float a0 = o[db][0] * inv, a1 = o[db][1] * inv, a2 = o[db][2] * inv, a3 = o[db][3] * inv;
      if constexpr (BF16) {
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.out) + orow + d) =
            u32x2{pack_bf16x2(a0, a1), pack_bf16x2(a2, a3)};
      } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + orow + d) = f32x4{a0, a1, a2, a3};
      }
    }
    if (p.lse && grp == 0) p.lse[(int64_t)t * p.Hq + h] = lse2 * kLn2;
  } else {
    const int64_t prow = (((int64_t)sp * p.T + t) * p.Hq + h);
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      const int d = db * 16 + grp * 4;
      *reinterpret_cast<f32x4*>(p.part_o + prow * D + d) = o[db] * inv;
    }
    if (grp == 0) p.part_lse[prow] = lse2;
  }
}

// One thread per (row, head, d); rows whose sequence had a single chunk were
// finished by pass 1.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void decode_merge_kernel(AttnParams p) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)p.T * p.Hq * D;
  if (idx >= total) return;
  const int d = (int)(idx % D);
  const int64_t th = idx / D;            // t * Hq + h
  const int t = (int)(th / p.Hq);
  const int Lk = p.lens_k[t];            // decode: row t belongs to sequence t
  const int nsplit = min((Lk + p.chunk - 1) / p.chunk, p.max_splits);
  if (nsplit <= 1) return;
  const int64_t plane = (int64_t)p.T * p.Hq;
  float M = kMaskedScore;
  for (int i = 0; i < nsplit; ++i) M = fmaxf(M, p.part_lse[i * plane + th]);
  float wsum = 0.f, acc = 0.f;
  for (int i = 0; i < nsplit; ++i) {
    const float w = __builtin_amdgcn_exp2f(p.part_lse[i * plane + th] - M);
    wsum += w;
    acc += w * p.part_o[(i * plane + th) * D + d];
  }
  const float val = acc / wsum;
  if constexpr (BF16) {
    reinterpret_cast<__bf16*>(p.out)[th * D + d] = (__bf16)val;
  } else {
    static_cast<float*>(p.out)[th * D + d] = val;
  }
  if (p.lse && d == 0) p.lse[th] = (M + __builtin_amdgcn_logf(wsum)) * kLn2;
}

template <int D, bool BF16>
static hipError_t launch_decode_t(const AttnParams& p, hipStream_t s) {
  hipLaunchKernelGGL((decode_split_kernel<D, BF16>), dim3(p.max_splits, p.Hkv, p.B), dim3(64), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.max_splits <= 1) return e;
  const int64_t total = (int64_t)p.T * p.Hq * D;
  hipLaunchKernelGGL((decode_merge_kernel<D, BF16>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_decode(const AttnParams& p, DType dt, int D, hipStream_t s) {
  if (dt == DType::BF16) return D == 64 ? launch_decode_t<64, true>(p, s) : launch_decode_t<128, true>(p, s);
  return D == 64 ? launch_decode_t<64, false>(p, s) : launch_decode_t<128, false>(p, s);
}

}  // namespace kvs
