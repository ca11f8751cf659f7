// Tree- or causal-masked verify attention on MFMA (gfx950).
//
// One workgroup per (batch row, head); wave w owns query rows 16w..16w+15.
// Keys stream in tiles of 32 from the cache into two LDS buffers (K and V
// row-major), with the next tile's global loads in flight while the current
// tile is multiplied, and one barrier per tile; at 120 VGPRs and 36 KB of
// LDS, four workgroups share a compute unit.  The V^T operand is formed on
// the way out of LDS by the transposing read ds_read_b64_tr_b16.  Per tile
// and wave:
//
//   S^T[32 keys x 16 queries] = K_tile . Q^T    2 key blocks x 4 d-steps of
//                                               v_mfma_f32_16x16x32_bf16
//   online softmax per query column (log2 domain), mask from a 64-bit
//   ancestor set per query for the keys in [L, L+N)
//   O^T[128 d x 16 queries] += V^T . P^T        8 d blocks x 1 key-step
//
// Keeping keys (and d) on the M side of both products puts every query in
// one lane column of the accumulator, so the running max, the rescale of O
// and the row sum need no cross-lane traffic except one 4-way combine at the
// end.  The key order inside a key-step is permuted identically on both
// operands of the P.V product so that P can be fed from the S accumulator
// registers directly.
//
// The pass is HBM-bound (64 flop per byte of K/V against a bf16 ridge near
// 312), so the matrix cores are used because the product is dense, not to
// reach their peak.  Mask semantics: kwkr.cn/news/620872 §2.1 (causal verify),
// cf-1.com/news/5632551 §5.4 and the lonae tree-attention paragraphs (tree mask).
#include <hip/hip_ext.h>

#include "sv_common.h"
#include "sv_internal.h"

namespace sv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kKT = 32;               // keys per tile
constexpr int kKB = kKT / 16;         // 16-key blocks per tile
constexpr int kKS = kKT / 32;         // 32-key steps of the P.V product
constexpr int kTileVecs = kKT * kD * 2 / 16 / 256;   // 16-byte loads per thread per tile and cache
constexpr int kKsStride = kD + 8;     // bf16 per K row in LDS (16 B pad)
// bf16 per V row in LDS: 72 dwords, so the four rows x 32 bytes that one
// 16-lane transposing read touches fall on 32 distinct banks
constexpr int kVsStride = kD + 16;

typedef short v4i16_t __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16, per group of 16 lanes: lane j receives element (j & 3)
// of the 4-element blocks addressed by lanes 4 e + (j >> 2), e = 0..3.  With
// lane i addressing row key0 + (i >> 2), column d0 + 4 (i & 3), lane j thus
// receives V[key0 + e][d0 + j] for e = 0..3: four consecutive keys of one
// column, as the MFMA A operand wants them.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  const v4i16_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (v4i16_t __attribute__((address_space(3)))*)p);
  return __builtin_bit_cast(uint2, r);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats to packed bf16, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void attn_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2 * kKT * kKsStride];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2 * kKT * kVsStride];
  __shared__ unsigned long long s_anc[kMaxNodes];
  __shared__ int s_L, s_ok;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int bh = blockIdx.x;
  const int b = bh / a.H;
  const int N = a.N;
  const long long headKV = (long long)bh * a.S_max * kD;
  const long long headQ = (long long)bh * N * kD;

  if (tid == 0) {
    const int L = a.prefix_len[b];
    s_L = L;
    s_ok = L >= 0 && (long long)L + N <= (long long)a.S_max;
  }
  if (tid < N) {
    unsigned long long m = 0ull;
    if (a.parents) {
      const int* par = a.parents + (long long)b * N;
      int j = tid;
      for (int steps = 0; steps < kMaxNodes && j >= 0; ++steps) {
        m |= 1ull << j;
        if (j == 0) break;
        const int p = par[j];
        if (p < 0 || p >= j) break;  // malformed parent: stop the walk
        j = p;
      }
    } else {
      m = ~0ull >> (63 - tid);       // chain: every earlier new token
    }
    s_anc[tid] = m;
  }
  __syncthreads();
  const int L = s_L;
  if (!s_ok) {
    for (int i = tid; i < N * kD; i += kThreads) a.out[headQ + i] = 0;
    if (a.lse && tid < N) a.lse[(long long)bh * N + tid] = __builtin_nanf("");
    return;
  }

  const int g = lane >> 4, col = lane & 15;
  const int qi = w * 16 + col;
  const bool qvalid = qi < N;
  bf16x8_t qop[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (qvalid) u = *(const uint4*)(a.q + headQ + (long long)qi * kD + ks * 32 + 8 * g);
    qop[ks] = as_bf16x8(u);
  }
  const unsigned long long anc = qvalid ? s_anc[qi] : 0ull;

  f32x4_t o[8];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) o[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_huge_valf();
  float l_run = 0.0f;  // this lane's share of the row sum

  const int total = L + N;
  const int n_tiles = (total + kKT - 1) / kKT;
  // The next tile's loads are in flight in registers while the current tile
  // is multiplied out of one of the two LDS buffers.  Keys past the end load
  // the last key (finite, masked to weight 0), so that no load sits behind a
  // branch: a load whose value crosses a branch join is waited for there,
  // which would drain the prefetch.
  u32x4_t kA[kTileVecs], vA[kTileVecs];
  auto load_tile = [&](u32x4_t (&kr)[kTileVecs], u32x4_t (&vr)[kTileVecs], int t) {
    t = min(t, n_tiles - 1);
#pragma unroll
    for (int j = 0; j < kTileVecs; ++j) {
      const int ci = j * kThreads + tid;
      const int key = ci >> 4, d0 = (ci & 15) * 8;
      const int gk = min(t * kKT + key, total - 1);
      // the cache rows are read once: non-temporal loads
      kr[j] = __builtin_nontemporal_load((const u32x4_t*)(a.k + headKV + (long long)gk * kD + d0));
      vr[j] = __builtin_nontemporal_load((const u32x4_t*)(a.v + headKV + (long long)gk * kD + d0));
    }
  };
  auto store_tile = [&](const u32x4_t (&kr)[kTileVecs], const u32x4_t (&vr)[kTileVecs], int buf) {
    uint16_t* ks = Ks + buf * (kKT * kKsStride);
    uint16_t* vs = Vs + buf * (kKT * kVsStride);
#pragma unroll
    for (int j = 0; j < kTileVecs; ++j) {
      const int ci = j * kThreads + tid;
      const int key = ci >> 4, d0 = (ci & 15) * 8;
      *(u32x4_t*)&ks[key * kKsStride + d0] = kr[j];
      *(u32x4_t*)&vs[key * kVsStride + d0] = vr[j];
    }
  };

  // One tile out of LDS buffer `buf`.
  auto compute_tile = [&](int t, int buf) {
    const uint16_t* ks = Ks + buf * (kKT * kKsStride);
    const uint16_t* vs = Vs + buf * (kKT * kVsStride);
    f32x4_t s[kKB];
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
      s[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks_ = 0; ks_ < 4; ++ks_) {
        const uint4 ku = *(const uint4*)&ks[(kb * 16 + col) * kKsStride + ks_ * 32 + 8 * g];
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ku), qop[ks_], s[kb], 0, 0, 0);
      }
    }

    const int tile0 = t * kKT;
    const bool need_mask = tile0 + kKT > L;
    float tmax = -__builtin_huge_valf();
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = s[kb][i] * a.scale_log2;
        if (need_mask) {
          const int kk = tile0 + kb * 16 + 4 * g + i;
          bool ok = kk < L;
          if (!ok && kk < total) ok = (anc >> (kk - L)) & 1ull;
          x = ok ? x : -__builtin_huge_valf();
        }
        s[kb][i] = x;
        tmax = fmaxf(tmax, x);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = m_new == -__builtin_huge_valf() ? 0.0f : m_new;
    const float alpha = exp2_hw(m_run - m_use);
    float psum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = exp2_hw(s[kb][i] - m_use);
        s[kb][i] = p;
        psum += p;
      }
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // the running maxima rarely move once the first tiles are in
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) o[mb] *= alpha;
    }

#pragma unroll
    for (int ks2 = 0; ks2 < kKS; ++ks2) {
      // logical keys 8g..8g+7 of this key-step = physical keys
      // 32*ks2 + 4g + {0..3} and 32*ks2 + 16 + 4g + {0..3}
      const uint4 pu = make_uint4(pack_bf16x2(s[2 * ks2][0], s[2 * ks2][1]),
                                  pack_bf16x2(s[2 * ks2][2], s[2 * ks2][3]),
                                  pack_bf16x2(s[2 * ks2 + 1][0], s[2 * ks2 + 1][1]),
                                  pack_bf16x2(s[2 * ks2 + 1][2], s[2 * ks2 + 1][3]));
      const bf16x8_t pop = as_bf16x8(pu);
      // V rows of the keys 32 ks2 + 4 g + {0..3} and 32 ks2 + 16 + 4 g + {0..3}
      const uint16_t* vlo = &vs[(ks2 * 32 + 4 * g + (col >> 2)) * kVsStride + 4 * (col & 3)];
      const uint16_t* vhi = vlo + 16 * kVsStride;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        const uint2 lo = lds_read_tr16(vlo + mb * 16);
        const uint2 hi = lds_read_tr16(vhi + mb * 16);
        const uint4 vu = make_uint4(lo.x, lo.y, hi.x, hi.y);
        o[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vu), pop, o[mb], 0, 0, 0);
      }
    }
  };

  // Tile t is multiplied out of LDS buffer t mod 2.  After it, tile t + 1
  // goes from the registers to the other buffer (last read for tile t - 1,
  // which every wave finished before the previous barrier), the registers
  // take tile t + 2, and one barrier publishes tile t + 1.  (Two 64-key tiles
  // in flight behind the multiplied one, two workgroups per compute unit:
  // 717 us at B=64, H=32, L=4096; this form: 696 us.)
  load_tile(kA, vA, 0);
  store_tile(kA, vA, 0);
  load_tile(kA, vA, 1);
  __syncthreads();
  for (int t = 0;; ++t) {
    compute_tile(t, t & 1);
    if (t + 1 >= n_tiles) break;
    store_tile(kA, vA, (t + 1) & 1);
    load_tile(kA, vA, t + 2);
    __syncthreads();
  }

  float l = l_run + __shfl_xor(l_run, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (qvalid) {
    const float inv = 1.0f / l;
    uint16_t* orow = a.out + headQ + (long long)qi * kD;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const uint2 pk = make_uint2(pack_bf16x2(o[mb][0] * inv, o[mb][1] * inv),
                                  pack_bf16x2(o[mb][2] * inv, o[mb][3] * inv));
      *(uint2*)(orow + mb * 16 + 4 * g) = pk;
    }
    if (a.lse && g == 0)
      a.lse[(long long)bh * N + qi] = (m_run + __log2f(l)) * 0.69314718055994531f;
  }
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t st, hipEvent_t ev_start, hipEvent_t ev_stop) {
  const dim3 grid((unsigned)((long long)a.B * a.H)), block(kThreads);
  if (ev_start && ev_stop)
    hipExtLaunchKernelGGL(attn_kernel, grid, block, 0, st, ev_start, ev_stop, 0, a);
  else
    attn_kernel<<<grid, block, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace sv
