// fa_decode.hip — incremental decode against a paged KV cache on gfx950.
//
// Page "FlashAttention 实战指南：如何把训练内存省 20 倍、速度提 4 倍", section
// "增量解码场景flash_attn_with_kvcache": each decode step appends the new K and V
// to the cache and attends in place; rotary_cos/rotary_sin apply a built-in
// rotary embedding; cache_seqlens marks each sample's valid length;
// block_table turns on a paged cache; num_splits cuts the keys into pieces
// to balance latency for small batches with long contexts.
//
// Split kernel: one work-group per (sequence, K/V head, split).  A split is a
// contiguous range of pages.  Its 4 waves take 32-key tiles round robin:
//   * the K tile goes HBM -> VGPR straight into the A operand of
//     S^T = K Q^T (one key row per lane, natural order);
//   * all query heads of the group (Hq / Hkv <= 32) are the 32 columns of the
//     B operand, so every K/V byte is read once for the whole group;
//   * the rotated query is split into a 16-bit high part and a 16-bit
//     remainder and both are multiplied, so rounding the rotated query to
//     16 bits costs no accuracy in the scores;
//   * V goes through a wave-private LDS tile and is read back transposed as
//     the A operand of O^T += V^T P^T;
//   * the tile holding position cache_seqlens[b] takes the rotated k_new and
//     v_new from registers and the same lanes write them to the cache slot,
//     so no other work-group ever reads that slot.
// The 4 waves' (max, sum, O) states are merged exactly in LDS.  With one
// split the kernel writes the final output; otherwise it writes float32
// partials (O_s normalised, LSE_s) that the combine kernel merges with
//   M = max_s LSE_s,  LSE = M + ln sum_s e^{LSE_s - M},  O = sum_s e^{LSE_s - LSE} O_s.
#include "fa_device.h"
#include "fa_host.h"

namespace fa {

struct DecParams {
  const uint16_t* q;
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* k_cache;
  uint16_t* v_cache;
  const int* cache_seqlens;
  const int* block_table;
  int max_blocks, page_size;
  const float* cos;
  const float* sin;
  int rotary_dim;
  uint16_t* out;
  float* lse;
  float* ws_o;
  float* ws_lse;
  int B, Hq, Hkv, G, num_splits;
  float scale_log2;
};

// Rotated 8-element chunk `ch` of a row (16-bit storage) as 8 floats.
template <int D, int DT>
__device__ __forceinline__ void rotate_chunk(const uint16_t* row, int ch, int pos, const DecParams& p, float out[8]) {
  const u32x4 a = gload128(row + ch * 8);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    out[2 * e] = to_f32<DT>((uint16_t)(a[e] & 0xffff));
    out[2 * e + 1] = to_f32<DT>((uint16_t)(a[e] >> 16));
  }
  const int rd = p.rotary_dim;
  if (rd == 0 || p.cos == nullptr) return;
  const int half = rd / 2;
  const int d0 = ch * 8;
  if (d0 >= rd) return;
  const bool first = d0 < half;
  const int pch = first ? ch + half / 8 : ch - half / 8;
  const u32x4 b = gload128(row + pch * 8);
  const int fi0 = first ? d0 : d0 - half;  // frequency index of element 0
  const float* cr = p.cos + (int64_t)pos * half + fi0;
  const float* sr = p.sin + (int64_t)pos * half + fi0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint16_t pb = (uint16_t)((e & 1) ? (b[e >> 1] >> 16) : (b[e >> 1] & 0xffff));
    const float y = to_f32<DT>(pb);
    const float c = cr[e], s = sr[e];
    out[e] = first ? (out[e] * c - y * s) : (out[e] * c + y * s);
  }
}

template <int DT>
__device__ __forceinline__ u32x4 pack8(const float x[8]) {
  u32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = pack2<DT>(x[2 * e], x[2 * e + 1]);
  return r;
}

template <int DT>
__device__ __forceinline__ float lo16(uint32_t v) { return to_f32<DT>((uint16_t)(v & 0xffff)); }
template <int DT>
__device__ __forceinline__ float hi16(uint32_t v) { return to_f32<DT>((uint16_t)(v >> 16)); }

template <int D, int DT>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(DecParams p) {
  constexpr int BK = 32;  // keys per wave tile
  constexpr int KC = D / 16, DB = D / 32;
  constexpr int VT = BK * D * 2;  // bytes of one wave's V tile
  __shared__ __attribute__((aligned(16))) char smem[4 * VT + 2 * 4 * 32 * 4];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hf = lane >> 5, r = lane & 31;
  const uint32_t tb = tr_base<D>(lane);
  const int s_id = blockIdx.x % p.num_splits;
  const int hkv = (blockIdx.x / p.num_splits) % p.Hkv;
  const int b = blockIdx.x / (p.num_splits * p.Hkv);

  const int L = p.cache_seqlens[b];
  const bool append = p.k_new != nullptr;
  const int n_keys = L + (append ? 1 : 0);
  const int page = p.page_size;
  const int n_pages = (n_keys + page - 1) / page;
  const int per = (n_pages + p.num_splits - 1) / p.num_splits;
  const int p_lo = s_id * per;
  const int p_hi = min(n_pages, p_lo + per);
  const int k_lo = p_lo * page;
  const int k_hi = min(p_hi * page, n_keys);

  // ---- query fragment (B operand, column = query head of the group) ----
  const int hq = hkv * p.G + r;
  const bool col_ok = r < p.G;
  const uint16_t* qrow = p.q + ((int64_t)b * p.Hq + hq) * D;
  u32x4 qhi[KC], qlo[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    if (col_ok) {
      float x[8], rem[8];
      rotate_chunk<D, DT>(qrow, 2 * c + hf, L, p, x);
      qhi[c] = pack8<DT>(x);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        rem[2 * e] = x[2 * e] - lo16<DT>(qhi[c][e]);
        rem[2 * e + 1] = x[2 * e + 1] - hi16<DT>(qhi[c][e]);
      }
      qlo[c] = pack8<DT>(rem);
    } else {
      qhi[c] = u32x4{0, 0, 0, 0};
      qlo[c] = u32x4{0, 0, 0, 0};
    }
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) oacc[d] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;
  char* vt = smem + w * VT;

  if (k_lo < k_hi) {
    const int t_lo = k_lo / BK, t_hi = (k_hi + BK - 1) / BK;
    const int64_t cap = (int64_t)p.max_blocks * page;
    for (int t = t_lo + w; t < t_hi; t += 4) {
      const int j0 = t * BK;
      const int j = j0 + r;  // key row this lane loads
      int64_t rowoff = 0;
      if (p.block_table) {
        const int phys = p.block_table[(int64_t)b * p.max_blocks + j0 / page];
        rowoff = (((int64_t)phys * page + (j % page)) * p.Hkv + hkv) * D;
      } else {
        rowoff = (((int64_t)b * cap + j) * p.Hkv + hkv) * D;
      }
      u32x4 ka[KC], va[KC];
      if (append && j == L) {
        const uint16_t* knr = p.k_new + ((int64_t)b * p.Hkv + hkv) * D;
        const uint16_t* vnr = p.v_new + ((int64_t)b * p.Hkv + hkv) * D;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          float x[8];
          rotate_chunk<D, DT>(knr, 2 * c + hf, L, p, x);
          ka[c] = pack8<DT>(x);
          va[c] = gload128(vnr + (2 * c + hf) * 8);
          gstore128(p.k_cache + rowoff + (2 * c + hf) * 8, ka[c]);
          gstore128(p.v_cache + rowoff + (2 * c + hf) * 8, va[c]);
        }
      } else if (j < n_keys) {
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          ka[c] = gload128(p.k_cache + rowoff + (2 * c + hf) * 8);
          va[c] = gload128(p.v_cache + rowoff + (2 * c + hf) * 8);
        }
      } else {
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          ka[c] = u32x4{0, 0, 0, 0};
          va[c] = u32x4{0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int c = 0; c < KC; ++c) lds_write128(vt, tile_off<D>(r, 2 * c + hf), va[c]);
      asm volatile("" ::: "memory");  // the wave reads its own V tile below

      f32x16 s = f32x16{};
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        s = mfma32<DT>(ka[c], qhi[c], s);
        s = mfma32<DT>(ka[c], qlo[c], s);
      }
      const bool ragged = j0 + BK > n_keys;
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (ragged && j0 + frag_row(i, hf) >= n_keys) s[i] = -INFINITY;
        mx = fmaxf(mx, s[i]);
      }
      mx = fmaxf(mx, xor32(mx));
      const float m_new = fmaxf(m_run, mx * p.scale_log2);
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float lsum = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = fast_exp2(fmaf(s[i], p.scale_log2, -m_use));
        s[i] = pv;
        lsum += pv;
      }
      l_run = fmaf(l_run, alpha, lsum);
      m_run = m_new;
#pragma unroll
      for (int d = 0; d < DB; ++d) oacc[d] *= alpha;
#pragma unroll
      for (int mk = 0; mk < 2; ++mk) {
        const u32x4 pb = pack_frag_half<DT>(s, mk);
#pragma unroll
        for (int d = 0; d < DB; ++d) oacc[d] = mfma32<DT>(lds_At<D>(vt + (16 * mk) * (D * 2), tb, d), pb, oacc[d]);
      }
    }
  }

  // ---- merge the 4 waves: M = max m_w, each wave scaled by 2^(m_w - M) ----
  float* mbuf = reinterpret_cast<float*>(smem + 4 * VT);  // [4][32]
  float* lbuf = mbuf + 4 * 32;                            // [4][32]
  const float l_w = l_run + xor32(l_run);
  if (hf == 0) {
    mbuf[w * 32 + r] = m_run;
    lbuf[w * 32 + r] = l_w;
  }
  __syncthreads();  // also ends every wave's use of its V tile
  float M = -INFINITY;
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, mbuf[ww * 32 + r]);
  const float M_use = (M == -INFINITY) ? 0.0f : M;
  const float fw = fast_exp2(m_run - M_use);
  // O^T fragments accumulate into obuf[d][32] (float), one wave after another
  float* obuf = reinterpret_cast<float*>(smem);
  for (int ww = 0; ww < 4; ++ww) {
    if (w == ww) {
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int dd = 32 * d + frag_row(i, hf);
          const float v = oacc[d][i] * fw;
          obuf[dd * 32 + r] = (ww == 0) ? v : obuf[dd * 32 + r] + v;
        }
    }
    __syncthreads();
  }
  // ---- write: each thread handles (column, d) pairs ----
  for (int idx = tid; idx < p.G * D; idx += 256) {
    const int col = idx / D, d = idx % D;
    const int h = hkv * p.G + col;
    // merged max and sum of this column (4 terms)
    float Mc = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) Mc = fmaxf(Mc, mbuf[ww * 32 + col]);
    const float Mcu = (Mc == -INFINITY) ? 0.0f : Mc;
    float lc = 0.0f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) lc += lbuf[ww * 32 + col] * fast_exp2(mbuf[ww * 32 + col] - Mcu);
    const float o = lc > 0.0f ? obuf[d * 32 + col] / lc : 0.0f;
    if (p.num_splits == 1) {
      uint16_t* orow = p.out + ((int64_t)b * p.Hq + h) * D;
      const uint32_t pk = pack2<DT>(o, 0.0f);
      orow[d] = (uint16_t)(pk & 0xffff);
      if (d == 0 && p.lse) p.lse[(int64_t)b * p.Hq + h] = lc > 0.0f ? (Mc + fast_log2(lc)) * kLn2 : INFINITY;
    } else {
      const int64_t pi = ((int64_t)b * p.Hq + h) * p.num_splits + s_id;
      p.ws_o[pi * D + d] = o;
      if (d == 0) p.ws_lse[pi] = lc > 0.0f ? (Mc + fast_log2(lc)) * kLn2 : -INFINITY;
    }
  }
}

// One wave per (sequence, query head).
template <int D, int DT>
__global__ __launch_bounds__(64) void decode_combine_kernel(DecParams p) {
  const int bh = blockIdx.x;  // b * Hq + h
  const int lane = threadIdx.x;
  const int S = p.num_splits;
  const float* ls = p.ws_lse + (int64_t)bh * S;
  float M = -INFINITY;
  for (int s = lane; s < S; s += 64) M = fmaxf(M, ls[s]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, __shfl_xor(M, m, 64));
  const float Mu = (M == -INFINITY) ? 0.0f : M;
  float sum = 0.0f;
  for (int s = lane; s < S; s += 64) sum += __expf(ls[s] - Mu);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) sum += __shfl_xor(sum, m, 64);
  const bool empty = !(sum > 0.0f);
  const float L = empty ? INFINITY : Mu + __logf(sum);
  for (int d = lane; d < D; d += 64) {
    float o = 0.0f;
    if (!empty) {
      for (int s = 0; s < S; ++s) {
        const float wgt = __expf(ls[s] - L);
        o = fmaf(wgt, p.ws_o[((int64_t)bh * S + s) * D + d], o);
      }
    }
    const uint32_t pk = pack2<DT>(o, 0.0f);
    p.out[(int64_t)bh * D + d] = (uint16_t)(pk & 0xffff);
  }
  if (lane == 0 && p.lse) p.lse[bh] = L;
}

template <int D, int DT>
static int launch_decode(const DecParams& p, hipStream_t st) {
  const long long nwg = (long long)p.B * p.Hkv * p.num_splits;
  if (nwg > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
  prof_before(FA_KERNEL_DECODE_SPLIT, st);
  hipLaunchKernelGGL((decode_split_kernel<D, DT>), dim3((int)nwg), dim3(256), 0, st, p);
  prof_after(FA_KERNEL_DECODE_SPLIT, st);
  if (p.num_splits > 1) {
    prof_before(FA_KERNEL_DECODE_COMBINE, st);
    hipLaunchKernelGGL((decode_combine_kernel<D, DT>), dim3(p.B * p.Hq), dim3(64), 0, st, p);
    prof_after(FA_KERNEL_DECODE_COMBINE, st);
  }
  return launch_status();
}

}  // namespace fa

using namespace fa;

extern "C" size_t fa_kvcache_workspace_size(int B, int Sq_new, int Hq, int D, int num_splits) {
  if (B < 1 || Sq_new < 1 || Hq < 1 || D < 1 || num_splits <= 1) return 0;
  const size_t parts = (size_t)B * Sq_new * Hq * num_splits;
  return align_up(parts * D * sizeof(float), 256) + align_up(parts * sizeof(float), 256);
}

extern "C" int fa_fwd_kvcache(const void* q, const void* k_new, const void* v_new,
                              void* k_cache, void* v_cache, const int* cache_seqlens,
                              const int* block_table, int max_blocks_per_seq, int page_size,
                              const float* rotary_cos, const float* rotary_sin, int rotary_dim,
                              void* out, float* lse,
                              int B, int Sq_new, int Hq, int Hkv, int D, int dtype,
                              float scale, int causal, int window_left, int window_right, float softcap,
                              const float* alibi_slopes, int num_splits,
                              void* workspace, size_t workspace_bytes, void* stream) {
  (void)causal;
  int st = check_common(Hq, Hkv, D, dtype, scale, window_left, window_right, softcap);
  if (st) return st;
  if (B < 1 || Sq_new < 1 || num_splits < 1 || max_blocks_per_seq < 1) return FA_ERR_INVALID_ARG;
  if (page_size < 32 || page_size % 32 != 0) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) return FA_ERR_INVALID_ARG;
  if (!aligned4(cache_seqlens)) return FA_ERR_INVALID_ARG;
  if ((k_new == nullptr) != (v_new == nullptr)) return FA_ERR_INVALID_ARG;
  if (!opt_aligned16(k_new) || !opt_aligned16(v_new)) return FA_ERR_INVALID_ARG;
  if (block_table && !aligned4(block_table)) return FA_ERR_INVALID_ARG;
  if (lse && !aligned4(lse)) return FA_ERR_INVALID_ARG;
  if ((rotary_cos == nullptr) != (rotary_sin == nullptr)) return FA_ERR_INVALID_ARG;
  if (rotary_cos && (rotary_dim < 16 || rotary_dim % 16 != 0 || rotary_dim > D)) return FA_ERR_INVALID_ARG;
  if (rotary_cos && (!aligned4(rotary_cos) || !aligned4(rotary_sin))) return FA_ERR_INVALID_ARG;
  if (Sq_new != 1) return FA_ERR_UNSUPPORTED;
  if (window_left != -1 || window_right != -1 || softcap != 0.0f || alibi_slopes) return FA_ERR_UNSUPPORTED;
  if (Hq / Hkv > 32) return FA_ERR_UNSUPPORTED;
  const size_t need = fa_kvcache_workspace_size(B, Sq_new, Hq, D, num_splits);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace))) return FA_ERR_WORKSPACE;

  DecParams p{};
  p.q = (const uint16_t*)q;
  p.k_new = (const uint16_t*)k_new;
  p.v_new = (const uint16_t*)v_new;
  p.k_cache = (uint16_t*)k_cache;
  p.v_cache = (uint16_t*)v_cache;
  p.cache_seqlens = cache_seqlens;
  p.block_table = block_table;
  p.max_blocks = max_blocks_per_seq;
  p.page_size = page_size;
  p.cos = rotary_cos;
  p.sin = rotary_sin;
  p.rotary_dim = rotary_cos ? rotary_dim : 0;
  p.out = (uint16_t*)out;
  p.lse = lse;
  const size_t parts = (size_t)B * Sq_new * Hq * num_splits;
  p.ws_o = need ? (float*)workspace : nullptr;
  p.ws_lse = need ? (float*)((char*)workspace + align_up(parts * D * sizeof(float), 256)) : nullptr;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.num_splits = num_splits;
  p.scale_log2 = scale * kLog2e;
  hipStream_t s = (hipStream_t)stream;
  if (D == 128) {
    return dtype == FA_DTYPE_BF16 ? launch_decode<128, DT_BF16>(p, s) : launch_decode<128, DT_F16>(p, s);
  }
  return dtype == FA_DTYPE_BF16 ? launch_decode<64, DT_BF16>(p, s) : launch_decode<64, DT_F16>(p, s);
}
