// fa_bwd.hip — backward pass of exact tiled attention on gfx950.
//
// The attention weights are not stored by the forward pass; they are
// recomputed here from q, k and the saved log-sum-exp (page "FlashAttention
// 实战指南：如何把训练内存省 20 倍、速度提 4 倍", section "FlashAttention 的做法是三个手段配合":
// recomputation is cheaper than round trips through HBM).  With z the final
// logits, P = exp(z - LSE) and
//   dV = P^T dO,  dP = dO V^T,  dZ = P * (dP - rowsum(dO * O)),
//   dS = dZ * (1 - tanh^2(s/c)) with softcap c (else dZ),
//   dQ = scale dS K,  dK = scale dS^T Q.
//
// Two kernels, none with atomics, so every result is bitwise reproducible
// (the pages' deterministic=True option is therefore always satisfied):
//   1. dQ: one work-group per 128 query rows of one query head (same layout
//      as the forward); it first forms the row terms -delta_i =
//      -sum_d dO_id O_id and LSE_i log2(e) (float32) of its rows and stores
//      them for the dK/dV kernel, then recomputes S^T and dP^T per key tile
//      and accumulates dQ^T += K^T dS^T;
//   2. dK/dV (launched after dQ on the same stream): one work-group per 256
//      keys of one K/V head; each wave keeps 32 keys' K rows in VGPRs (their
//      V rows sit in LDS) and walks every query head of its group and every
//      query tile of 64 rows in a fixed order, with Q and dO tiles copied
//      into LDS by DMA.  S = Q K^T puts one key per lane, so dV^T += dO^T P
//      and dK^T += Q^T dS take P / dS straight from the accumulators.
// Both recompute kernels fit in 256 VGPRs, so two waves share each SIMD and
// one wave's exponentials overlap the other's matrix instructions.
#include <type_traits>

#include "fa_device.h"
#include "fa_host.h"

namespace fa {

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  float* dvec;  // workspace: row term -delta, same layout as lse
  float* lse2;  // workspace: lse * log2(e), same layout as lse
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  const int* cu_q;
  const int* cu_k;
  int Sq, Sk, Hq, g, total_q;
  // elements between consecutive tokens: q; k and v; o and dout; dq; dk and dv
  int q_rstride, k_rstride, o_rstride, dq_rstride, dkv_rstride;
  float scale, scale_log2, scale_over_cap, cap_log2, inv_cap_log2;
  const float* alibi;
  int wl, wr;
  int n_tiles, n_heads, n_batch, reverse, balanced;
  int group;  // balanced: pairs per XCD group (tile_id)
  const int* tiles;  // varlen tile list (entries x 2 ints), or NULL
  DropSpec drop; // DROP kernels only
};

// dK/dV work-group: waves of 32 keys each (two waves per SIMD) and query
// tile rows.  D = 256 runs 4 waves (one per SIMD: K 64, dK and dV 256
// registers) and 32-row query tiles so V rows plus two stages fit in LDS.
template <int D>
struct DkdvShape {
  static constexpr int NW = D >= 256 ? 4 : 8;
  static constexpr int BR = D >= 256 ? 32 : 64;
};

struct SeqBounds {
  int q_start, Sq, k_start, Sk;
};

__device__ __forceinline__ SeqBounds seq_bounds(const BwdParams& p, int b) {
  SeqBounds s;
  if (p.cu_q) {
    s.q_start = p.cu_q[b];
    s.Sq = p.cu_q[b + 1] - s.q_start;
    s.k_start = p.cu_k[b];
    s.Sk = p.cu_k[b + 1] - s.k_start;
  } else {
    s.q_start = b * p.Sq;
    s.Sq = p.Sq;
    s.k_start = b * p.Sk;
    s.Sk = p.Sk;
  }
  return s;
}

__device__ __forceinline__ int64_t row_index(const BwdParams& p, int b, int h, int q_start, int Sq, int i) {
  return p.cu_q ? (int64_t)h * p.total_q + q_start + i : ((int64_t)b * p.Hq + h) * Sq + i;
}

// --------------------------------------------------- logit transform ------
// Log2-domain logit of raw dot product s for query position ip, key j, when
// softcap or ALiBi is on (otherwise the scale is folded into the exponent).
template <bool SOFTCAP, bool ALIBI>
__device__ __forceinline__ float logit2(float s, int ip, int j, const BwdParams& p, float slope_log2) {
  float x = SOFTCAP ? p.cap_log2 * tanh_exp(s * p.scale_over_cap) : s * p.scale_log2;
  if constexpr (ALIBI) x -= slope_log2 * (float)abs(ip - j);
  return x;
}

// dS = dZ * (1 - tanh^2(s/c)) with softcap c; tanh is recovered from the
// log2 logit x = c log2(e) tanh(s/c) - ALiBi term.  Masked entries (p = 0,
// x = -inf) stay 0.
template <bool ALIBI>
__device__ __forceinline__ float softcap_grad(float ds, float pv, float x, int ip, int j, const BwdParams& p,
                                              float slope_log2) {
  float xt = x;
  if constexpr (ALIBI) xt += slope_log2 * (float)abs(ip - j);
  const float t = xt * p.inv_cap_log2;
  return pv > 0.0f ? ds * fmaf(-t, t, 1.0f) : 0.0f;
}

// --------------------------------------------------------------- dK / dV --
// Work-group = 256 keys of one K/V head, 8 waves of 32 keys (two per SIMD).
// K rows stay in VGPRs; V rows sit in LDS for the whole kernel (that frees
// the VGPRs two waves per SIMD need).  Query tiles of 64 rows (Q, dO, LSE,
// delta) are copied into LDS by DMA, double buffered; the copy of tile n+1
// runs under the matrix work of tile n.
// DG < D: head dim DG in memory, padded to D on chip (see fwd_kernel).
template <int D, int DT, bool SOFTCAP, bool ALIBI, bool DROP, int DG = D>
__global__ __launch_bounds__(64 * DkdvShape<D>::NW, 1) void bwd_dkdv_kernel(BwdParams p) {
  constexpr int NW = DkdvShape<D>::NW, BC = 32 * NW, BR = DkdvShape<D>::BR;
  constexpr int KC = D / 16, DB = D / 32;
  constexpr int TILE = BR * D * 2;
  // A stage: LSE and delta rows (64 floats each whatever BR is, one 4-byte
  // DMA per lane), then the Q and dO tiles.
  constexpr int ROWT = 2 * 64 * 4;
  constexpr int STAGE = ROWT + 2 * TILE;
  // Two stage buffers and the V rows of the work-group's keys (B operand of
  // dP = dO V^T): distinct arrays, so that reads of one are never ordered
  // behind the DMA into another.  Every wave addresses its V rows from the
  // one V array: a pointer chosen between two arrays at run time would let
  // the compiler assume it may alias a stage and wait for the next stage's
  // copy (vmcnt(0)) before the first V read of every tile.
  __shared__ __attribute__((aligned(1024))) char sm0[STAGE];
  __shared__ __attribute__((aligned(1024))) char sm1[STAGE];
  __shared__ __attribute__((aligned(1024))) char vsm[BC * D * 2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, known uniform
  const int g = lane >> 5, r = lane & 31;
  const uint32_t nb = nat_base<D>(lane);
  const uint32_t tb = tr_base<D>(lane);
  // causal: the first key tiles are seen by the most queries
  TileId tid3;
  if (p.tiles) {
    if (!tile_from_list(p.tiles, p.n_heads, tid3)) return;  // unused list entry
  } else {
    tid3 = tile_id(p.n_tiles, p.n_heads, p.n_batch, p.balanced != 0, false, p.group);
  }
  const int tk = tid3.t, hk = tid3.h, b = tid3.b;
  const SeqBounds sb = seq_bounds(p, b);
  const int k0 = tk * BC;
  if (k0 >= sb.Sk) return;
  const int Sq = sb.Sq, Sk = sb.Sk, off = Sk - Sq;
  const MaskSpec mask{p.wl, p.wr};

  const int kw0 = k0 + 32 * w;
  const int my_key = kw0 + r;
  const bool key_ok = my_key < Sk;
  const int64_t krow = (int64_t)(sb.k_start + my_key) * p.k_rstride + hk * DG;

  u32x4 kreg[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    const bool in = DG == D || (2 * c + g) * 8 < DG;
    kreg[c] = (key_ok && in) ? gload128(p.k + krow + (2 * c + g) * 8) : u32x4{0, 0, 0, 0};
  }
  zero_pad<D, BC, DG>(vsm, tid, 64 * NW);
  zero_pad<D, BR, DG>(sm0 + ROWT, tid, 64 * NW);
  zero_pad<D, BR, DG>(sm0 + ROWT + TILE, tid, 64 * NW);
  zero_pad<D, BR, DG>(sm1 + ROWT, tid, 64 * NW);
  zero_pad<D, BR, DG>(sm1 + ROWT + TILE, tid, 64 * NW);
  // this wave's 32 V rows
  const char* vw = vsm + (32 * w) * (D * 2);
  f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) {
    dkacc[d] = f32x16{};
    dvacc[d] = f32x16{};
  }

  // query rows that can see any key of this work-group
  const int k1 = min(k0 + BC, Sk) - 1;
  int i_lo = 0, i_hi = Sq;
  if (p.wr >= 0) i_lo = max(0, k0 - p.wr - off);
  if (p.wl >= 0) i_hi = min(Sq, k1 + p.wl - off + 1);
  if (i_lo < i_hi) {
    const int t_lo = i_lo / BR, nt = (i_hi + BR - 1) / BR - t_lo;
    const int n_iter = nt * p.g;
    auto issue = [&](int n, char* st) {
      const int hq = hk * p.g + n / nt;
      const int i0 = (t_lo + n % nt) * BR;
      const int64_t hoff = (int64_t)sb.q_start * p.q_rstride + (int64_t)hq * DG;
      const int64_t ooff = (int64_t)sb.q_start * p.o_rstride + (int64_t)hq * DG;
      dma_tile<D, BR, NW, true, DG>(st + ROWT, p.q + hoff, p.q_rstride, i0, Sq, w, lane);
      dma_tile<D, BR, NW, true, DG>(st + ROWT + TILE, p.dout + ooff, p.o_rstride, i0, Sq, w, lane);
      if (w < 2) {
        const float* src = (w == 0) ? p.lse2 : p.dvec;
        const int i = min(i0 + lane, Sq - 1);  // i0 < Sq, so i - i0 >= 0
        dma4(make_rsrc(src + row_index(p, b, hq, sb.q_start, Sq, i0)), (uint32_t)(i - i0) * 4u, st + w * 64 * 4);
      }
    };

    // One query tile: `st` holds tile n, `nxt` receives tile n + 1.
    auto step = [&](const char* st, char* nxt, int n) {
      if (n + 1 < n_iter) issue(n + 1, nxt);
      const uint32_t nbv = opaque(nb), tbv = opaque(tb);
      const int hq = hk * p.g + n / nt;
      const int i0 = (t_lo + n % nt) * BR;
      const char* qt = st + ROWT;
      const char* dot = st + ROWT + TILE;
      const float* lse2 = reinterpret_cast<const float*>(st);
      const float* dvs = lse2 + 64;
      const float slope_log2 = ALIBI ? p.alibi[hq] * kLog2e : 0.0f;
      const float fs = (SOFTCAP || ALIBI) ? 1.0f : p.scale_log2;
#pragma unroll
      for (int rb = 0; rb < BR / 32; ++rb) {
        const int r0 = i0 + 32 * rb;
        if (r0 >= Sq) break;
        int cls = classify(r0 + off, min(r0 + 31, Sq - 1) + off, kw0, kw0 + 31, Sk, mask);
        if (cls == 0) continue;
        if (r0 + 31 >= Sq) cls = 1;  // rows past the end hold a copy of the last row
        // S = Q K^T and dP = dO V^T: rows = 32 queries, columns = this wave's
        // keys.  Every phase below is one explicitly ordered block
        // (sched_barrier after every MFMA) whose LDS operands run in rings a
        // few MFMAs ahead of their use, so no MFMA waits for the full LDS
        // latency of its own operand.
        const char* qr = qt + (32 * rb) * (D * 2);
        const char* dr = dot + (32 * rb) * (D * 2);
        constexpr int R1 = KC > 2 ? 2 : 1;  // chunk steps in flight ahead
        constexpr int N2 = 4 * DB;          // dV and dK MFMAs
        constexpr int R2 = 3;               // transposed operands in flight
        auto op2 = [&](int i) -> u32x4 {
          const int mk = i / (2 * DB), d = (i >> 1) % DB;
          return lds_At<D>(((i & 1) ? qt : dot) + (32 * rb + 16 * mk) * (D * 2), tbv, d);
        };
        // dP accumulates onto -delta (stored negated), so it leaves the MFMAs
        // as dP - delta; with dropout the keep mask acts on dP alone
        f32x16 s = f32x16{}, dp = f32x16{};
        if constexpr (!DROP) {
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) {
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(dvs + 32 * rb + 8 * qd + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) dp[4 * qd + e] = d4[e];
          }
        }
        {
          u32x4 qa[R1 + 1], oa[R1 + 1], va[R1 + 1];
#pragma unroll
          for (int k = 0; k < R1; ++k) {
            qa[k] = lds_nat(qr, nbv, k);
            oa[k] = lds_nat(dr, nbv, k);
            va[k] = lds_nat(vw, nbv, k);
          }
#pragma unroll
          for (int c = 0; c < KC; ++c) {
            if (c + R1 < KC) {
              const int sl = (c + R1) % (R1 + 1);
              qa[sl] = lds_nat(qr, nbv, c + R1);
              oa[sl] = lds_nat(dr, nbv, c + R1);
              va[sl] = lds_nat(vw, nbv, c + R1);
            }
            s = mfma32<DT>(qa[c % (R1 + 1)], kreg[c], s);
            dp = mfma32<DT>(oa[c % (R1 + 1)], va[c % (R1 + 1)], dp);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // the first dV / dK operands load under the element-wise work
        u32x4 r2[R2];
#pragma unroll
        for (int i = 0; i < R2; ++i) r2[i] = op2(i);
        // logits, mask (rows past Sq hold a copy of the last row), P and dS
        if constexpr (SOFTCAP || ALIBI) {
#pragma unroll
          for (int ii = 0; ii < 16; ++ii) {
            const int ip = r0 + frag_row(ii, g) + off;
            s[ii] = logit2<SOFTCAP, ALIBI>(s[ii], ip, my_key, p, slope_log2);
          }
        }
        if (cls == 1) {
          const RangeTest rt = range_test(rows_for_key(key_ok, my_key, Sq, off, mask), r0 + 4 * g);
#pragma unroll
          for (int ii = 0; ii < 16; ++ii) s[ii] = in_range(rt, ii) ? s[ii] : -INFINITY;
        }
        // dropout: kept weights enter dV and dP (scaled once at the end / here)
        uint32_t kx[4];
        if constexpr (DROP) drop_words<true>(p.drop, (uint32_t)(b * p.Hq + hq), my_key, r0, lane, kx);
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse2 + 32 * rb + 8 * qd + 4 * g);
          f32x4 d4 = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
          if constexpr (DROP) d4 = *reinterpret_cast<const f32x4*>(dvs + 32 * rb + 8 * qd + 4 * g);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int ii = 4 * qd + e;
            const float pv = fast_exp2(fmaf(s[ii], fs, -l4[e]));
            bool keep = true;
            float dpv = dp[ii];
            if constexpr (DROP) {
              keep = drop_keep(kx, ii, p.drop.t);
              dpv = (keep ? dpv * p.drop.scale : 0.0f) + d4[e];
            }
            float ds = pv * dpv;
            if constexpr (SOFTCAP) {
              ds = softcap_grad<ALIBI>(ds, pv, s[ii], r0 + frag_row(ii, g) + off, my_key, p, slope_log2);
            }
            s[ii] = keep ? pv : 0.0f;
            dp[ii] = ds;
          }
        }
        // dV^T += dO^T P ;  dK^T += Q^T dS   (contraction over the 32 query rows)
        u32x4 pb[2], sb2[2];
#pragma unroll
        for (int mk = 0; mk < 2; ++mk) {
          pb[mk] = pack_frag_half<DT>(s, mk);
          sb2[mk] = pack_frag_half<DT>(dp, mk);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < N2; ++i) {
          const int mk = i / (2 * DB), d = (i >> 1) % DB;
          if (i & 1) dkacc[d] = mfma32<DT>(r2[i % R2], sb2[mk], dkacc[d]);
          else dvacc[d] = mfma32<DT>(r2[i % R2], pb[mk], dvacc[d]);
          if (i + R2 < N2) r2[i % R2] = op2(i + R2);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      dma_wait();
      __syncthreads();
    };

    // V rows past Sk hold a copy of the last row; their keys are masked
    const uint16_t* vsrc = p.v + (int64_t)sb.k_start * p.k_rstride + hk * DG;
    dma_tile<D, BC, NW, true, DG>(vsm, vsrc, p.k_rstride, k0, Sk, w, lane);
    issue(0, sm0);
    dma_wait();
    __syncthreads();
    int n = 0;
    for (; n + 1 < n_iter; n += 2) {
      step(sm0, sm1, n);
      step(sm1, sm0, n + 1);
    }
    if (n < n_iter) step(sm0, sm1, n);
  }

  if (key_ok) {
    const int64_t drow_off = (int64_t)(sb.k_start + my_key) * p.dkv_rstride + hk * DG;
    uint16_t* dkrow = p.dk + drow_off;
    uint16_t* dvrow = p.dv + drow_off;
#pragma unroll
    for (int d = 0; d < DB; ++d) {
      if (32 * d >= DG) continue;  // padded columns
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        u32x2 a, c;
        a[0] = pack2<DT>(dkacc[d][4 * qd + 0] * p.scale, dkacc[d][4 * qd + 1] * p.scale);
        a[1] = pack2<DT>(dkacc[d][4 * qd + 2] * p.scale, dkacc[d][4 * qd + 3] * p.scale);
        const float vs = DROP ? p.drop.scale : 1.0f;
        c[0] = pack2<DT>(dvacc[d][4 * qd + 0] * vs, dvacc[d][4 * qd + 1] * vs);
        c[1] = pack2<DT>(dvacc[d][4 * qd + 2] * vs, dvacc[d][4 * qd + 3] * vs);
        gstore64(dkrow + 32 * d + 8 * qd + 4 * g, a);
        gstore64(dvrow + 32 * d + 8 * qd + 4 * g, c);
      }
    }
  }
}

// ------------------------------------------------------------------ dQ ----
// Work-group = 128 query rows of one query head (4 waves of 32 rows), two
// work-groups per CU; K/V tiles of 64 keys are copied into LDS by DMA,
// double buffered.
template <int D, int DT, bool SOFTCAP, bool ALIBI, bool DROP, int DG = D>
__global__ __launch_bounds__(256, D >= 256 ? 1 : 2) void bwd_dq_kernel(BwdParams p) {
  constexpr int BR = 128, BC = 64;
  constexpr int KC = D / 16, DB = D / 32;
  constexpr int TILE = BC * D * 2;
  // two stage buffers (K tile then V tile), distinct arrays so that reads of
  // one are never ordered behind the DMA into the other
  __shared__ __attribute__((aligned(1024))) char sm0[2 * TILE];
  __shared__ __attribute__((aligned(1024))) char sm1[2 * TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index stays a per-lane value here: declared uniform (readfirstlane)
  // it changes register allocation enough to spill about 80 VGPRs
  const int w = tid >> 6;
  const int g = lane >> 5, r = lane & 31;
  const uint32_t nb = nat_base<D>(lane);
  const uint32_t tb = tr_base<D>(lane);
  // causal: the last query tiles see the most keys
  TileId tid3;
  if (p.tiles) {
    if (!tile_from_list(p.tiles, p.n_heads, tid3)) return;  // unused list entry
  } else {
    tid3 = tile_id(p.n_tiles, p.n_heads, p.n_batch, p.balanced != 0, p.reverse != 0, p.group);
  }
  const int tq = tid3.t, h = tid3.h, b = tid3.b;
  const SeqBounds sb = seq_bounds(p, b);
  const int q0 = tq * BR;
  if (q0 >= sb.Sq) return;
  const int Sq = sb.Sq, Sk = sb.Sk, off = Sk - Sq;
  const int hk = h / p.g;
  const MaskSpec mask{p.wl, p.wr};

  const int wrow0 = q0 + 32 * w;
  const int wrow1 = min(wrow0 + 31, Sq - 1);
  const int my_row = wrow0 + r;
  const bool row_ok = my_row < Sq;
  const int ip = my_row + off;
  const int64_t qrow = (int64_t)(sb.q_start + my_row) * p.q_rstride + h * DG;
  const int64_t orow = (int64_t)(sb.q_start + my_row) * p.o_rstride + h * DG;

  u32x4 qreg[KC], doreg[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    const bool in = row_ok && (DG == D || (2 * c + g) * 8 < DG);
    qreg[c] = in ? gload128(p.q + qrow + (2 * c + g) * 8) : u32x4{0, 0, 0, 0};
    doreg[c] = in ? gload128(p.dout + orow + (2 * c + g) * 8) : u32x4{0, 0, 0, 0};
  }
  zero_pad<D, BC, DG>(sm0, tid, 256);
  zero_pad<D, BC, DG>(sm0 + TILE, tid, 256);
  zero_pad<D, BC, DG>(sm1, tid, 256);
  zero_pad<D, BC, DG>(sm1 + TILE, tid, 256);
  // Row terms of this work-group's rows: -delta = -sum_d dO O (lane g sums
  // its half of the head dim, the two halves meet across lanes l, l ^ 32)
  // and the LSE in log2 units.  Both are stored for the dK/dV kernel, which
  // runs after this one on the same stream.
  float lse2 = INFINITY, ndelta = 0.0f;  // rows past the end: P = 0
  {
    float dacc = 0.0f;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const bool in = row_ok && (DG == D || (2 * c + g) * 8 < DG);
      const u32x4 o4 = in ? gload128(p.o + orow + (2 * c + g) * 8) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dacc = fmaf(to_f32<DT>((uint16_t)(o4[e] & 0xffff)), to_f32<DT>((uint16_t)(doreg[c][e] & 0xffff)), dacc);
        dacc = fmaf(to_f32<DT>((uint16_t)(o4[e] >> 16)), to_f32<DT>((uint16_t)(doreg[c][e] >> 16)), dacc);
      }
    }
    const float dsum = pair_sum32(dacc);
    if (row_ok) {
      const int64_t ri = row_index(p, b, h, sb.q_start, Sq, my_row);
      lse2 = p.lse[ri] * kLog2e;
      ndelta = -dsum;
      if (g == 0) {
        p.dvec[ri] = ndelta;
        p.lse2[ri] = lse2;
      }
    }
  }
  const float slope_log2 = ALIBI ? p.alibi[h] * kLog2e : 0.0f;
  const float fs = (SOFTCAP || ALIBI) ? 1.0f : p.scale_log2;

  f32x16 dqacc[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) dqacc[d] = f32x16{};

  const int qend = min(q0 + BR, Sq);
  int kv_lo = 0, kv_hi = Sk;
  if (p.wl >= 0) kv_lo = max(0, q0 + off - p.wl);
  if (p.wr >= 0) kv_hi = min(Sk, qend - 1 + off + p.wr + 1);
  const uint16_t* kbase = p.k + (int64_t)sb.k_start * p.k_rstride + hk * DG;
  const uint16_t* vbase = p.v + (int64_t)sb.k_start * p.k_rstride + hk * DG;

  if (kv_lo < kv_hi) {
    const int t_lo = kv_lo / BC, t_hi = (kv_hi + BC - 1) / BC;
    auto issue = [&](int t, char* kt) {
      dma_tile<D, BC, 4, false, DG>(kt, kbase, p.k_rstride, t * BC, Sk, w, lane);
      dma_tile<D, BC, 4, false, DG>(kt + TILE, vbase, p.k_rstride, t * BC, Sk, w, lane);
    };
    // One key tile: `kt` holds K and V of tile t, `nxt` receives tile t + 1.
    auto step = [&](const char* kt, char* nxt, int t) {
      const uint32_t nbv = opaque(nb), tbv = opaque(tb);
      const char* vt = kt + TILE;
      constexpr int RA = 4;  // natural-order operands in flight
      // operand i of the S / dP phase: K (even i) or V (odd i) rows of key
      // half i / (2 KC), chunk step (i / 2) % KC
      auto op_a = [&](int i) -> u32x4 {
        const int kb = i / (2 * KC), c = (i >> 1) % KC;
        return lds_nat(((i & 1) ? vt : kt) + (kb * 32) * (D * 2), nbv, c);
      };
      // the first operands are read before the copy of the next tile is
      // issued and the tile is classified, so their LDS latency overlaps that
      u32x4 ra0[RA];
#pragma unroll
      for (int i = 0; i < RA; ++i) ra0[i] = op_a(i);
      if (t + 1 < t_hi) issue(t + 1, nxt);
      const int j0 = t * BC;
      // keys past the end hold a copy of the last key: classify marks such tiles partial
      const int cls = (wrow0 < Sq) ? classify(wrow0 + off, wrow1 + off, j0, j0 + BC - 1, Sk, mask) : 0;
      // The tile body is written out twice, without and with the mask.  Both
      // are one explicitly ordered block (sched_barrier after every MFMA):
      //   S/dP of half 0, then S/dP of half 1 with the element-wise work of
      //   half 0 (P, dS) spread over its MFMAs, then dQ of half 0 with the
      //   element-wise work of half 1 spread over it, then dQ of half 1.
      // LDS operands run in rings a few MFMAs ahead of their use, so no MFMA
      // waits for the full LDS latency of its own operand.
      auto body = [&](auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
        constexpr int NA = 4 * KC;  // S and dP MFMAs of both halves
        constexpr int NB = 4 * DB;  // dQ MFMAs of both halves
        constexpr int RB = 3;       // transposed operands in flight
        auto op_b = [&](int i) -> u32x4 { return lds_At<D>(kt + (16 * (i / DB)) * (D * 2), tbv, i % DB); };
        f32x16 s[2], dp[2];
        uint32_t kx[2][4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          s[kb] = f32x16{};
          dp[kb] = f32x16{};
          if constexpr (DROP) drop_words<false>(p.drop, (uint32_t)(b * p.Hq + h), my_row, j0 + 32 * kb, lane, kx[kb]);
        }
        // element i of half kb: logit, mask (keys past Sk hold a copy of the
        // last key), P, and dS in place of dP
        const LaneRange kr = keys_for_row(row_ok, ip, Sk, mask);
        auto elem = [&](int kb, int i) {
          const int j = j0 + 32 * kb + frag_row(i, g);
          float x = s[kb][i];
          if constexpr (SOFTCAP || ALIBI) x = logit2<SOFTCAP, ALIBI>(x, ip, j, p, slope_log2);
          if constexpr (MASKED) x = in_range(range_test(kr, j0 + 32 * kb + 4 * g), i) ? x : -INFINITY;
          const float pv = fast_exp2(fmaf(x, fs, -lse2));
          float dpv = dp[kb][i];
          if constexpr (DROP) dpv = drop_keep(kx[kb], i, p.drop.t) ? dpv * p.drop.scale : 0.0f;
          float ds = pv * (dpv + ndelta);
          if constexpr (SOFTCAP) ds = softcap_grad<ALIBI>(ds, pv, x, ip, j, p, slope_log2);
          dp[kb][i] = ds;
        };
        u32x4 db[4];
        u32x4 ra[RA], rb[RB];
#pragma unroll
        for (int i = 0; i < RA; ++i) ra[i] = ra0[i];
#pragma unroll
        for (int i = 0; i < NA; ++i) {
          const int kb = i / (2 * KC), c = (i >> 1) % KC;
          if (i & 1) dp[kb] = mfma32<DT>(ra[i % RA], doreg[c], dp[kb]);
          else s[kb] = mfma32<DT>(ra[i % RA], qreg[c], s[kb]);
          if (i + RA < NA) ra[i % RA] = op_a(i + RA);
          else if (i + RA - NA < RB) rb[i + RA - NA] = op_b(i + RA - NA);
          if (kb == 1) {
            const int jj = i - 2 * KC;
#pragma unroll
            for (int e = 16 * jj / (2 * KC); e < 16 * (jj + 1) / (2 * KC); ++e) elem(0, e);
            if (16 * (jj + 1) / (2 * KC) >= 8 && 16 * jj / (2 * KC) < 8) db[0] = pack_frag_half<DT>(dp[0], 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        db[1] = pack_frag_half<DT>(dp[0], 1);
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const int mk = i / DB, d = i % DB;
          dqacc[d] = mfma32<DT>(rb[i % RB], db[mk], dqacc[d]);
          if (i + RB < NB) rb[i % RB] = op_b(i + RB);
          if (mk < 2) {
            const int jj = i;
#pragma unroll
            for (int e = 16 * jj / (2 * DB); e < 16 * (jj + 1) / (2 * DB); ++e) elem(1, e);
            if (16 * (jj + 1) / (2 * DB) >= 8 && 16 * jj / (2 * DB) < 8) db[2] = pack_frag_half<DT>(dp[1], 0);
            if (jj == 2 * DB - 1) db[3] = pack_frag_half<DT>(dp[1], 1);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      if (cls == 2) body(std::false_type{});
      else if (cls == 1) body(std::true_type{});
      dma_wait();
      __syncthreads();
    };

    issue(t_lo, sm0);
    dma_wait();
    __syncthreads();
    int t = t_lo;
    for (; t + 1 < t_hi; t += 2) {
      step(sm0, sm1, t);
      step(sm1, sm0, t + 1);
    }
    if (t < t_hi) step(sm0, sm1, t);
  }

  if (row_ok) {
    uint16_t* drow = p.dq + (int64_t)(sb.q_start + my_row) * p.dq_rstride + h * DG;
#pragma unroll
    for (int d = 0; d < DB; ++d) {
      if (32 * d >= DG) continue;  // padded columns
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        u32x2 v2;
        v2[0] = pack2<DT>(dqacc[d][4 * qd + 0] * p.scale, dqacc[d][4 * qd + 1] * p.scale);
        v2[1] = pack2<DT>(dqacc[d][4 * qd + 2] * p.scale, dqacc[d][4 * qd + 3] * p.scale);
        gstore64(drow + 32 * d + 8 * qd + 4 * g, v2);
      }
    }
  }
}

// ------------------------------------------------------------- dispatch ---
template <int D, int DT, bool SC, bool AL, bool DR, int DG>
static void launch_main(const BwdParams& dkdv, const BwdParams& dq, int nwg_kv, int nwg_q, hipStream_t st) {
  // dQ first: it writes the row terms the dK/dV kernel reads
  if (nwg_q > 0) {
    prof_before(FA_KERNEL_BWD_DQ, st);
    hipLaunchKernelGGL((bwd_dq_kernel<D, DT, SC, AL, DR, DG>), dim3(nwg_q), dim3(256), 0, st, dq);
    prof_after(FA_KERNEL_BWD_DQ, st);
  }
  if (nwg_kv > 0) {
    prof_before(FA_KERNEL_BWD_DKDV, st);
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, DT, SC, AL, DR, DG>), dim3(nwg_kv), dim3(64 * DkdvShape<D>::NW), 0, st,
                       dkdv);
    prof_after(FA_KERNEL_BWD_DKDV, st);
  }
}

template <int D, int DT, bool SC, bool AL, int DG>
static void launch_main_d(const BwdParams& dkdv, const BwdParams& dq, int nwg_kv, int nwg_q, bool dr,
                          hipStream_t st) {
  if (dr) launch_main<D, DT, SC, AL, true, DG>(dkdv, dq, nwg_kv, nwg_q, st);
  else launch_main<D, DT, SC, AL, false, DG>(dkdv, dq, nwg_kv, nwg_q, st);
}

// D: the head dim on chip; DG: in memory (DG < D only for D = 96 on 128)
template <int D, int DT, int DG = D>
static void launch_all(const BwdParams& dkdv, const BwdParams& dq, int nwg_kv, int nwg_q, bool sc, bool al,
                       hipStream_t st) {
  const bool dr = dkdv.drop.t > 0;
  if (sc) {
    if (al) launch_main_d<D, DT, true, true, DG>(dkdv, dq, nwg_kv, nwg_q, dr, st);
    else launch_main_d<D, DT, true, false, DG>(dkdv, dq, nwg_kv, nwg_q, dr, st);
  } else {
    if (al) launch_main_d<D, DT, false, true, DG>(dkdv, dq, nwg_kv, nwg_q, dr, st);
    else launch_main_d<D, DT, false, false, DG>(dkdv, dq, nwg_kv, nwg_q, dr, st);
  }
}

// Keys per dK/dV work-group.
inline int dkdv_keys(int D) { return 32 * (D >= 256 ? DkdvShape<256>::NW : DkdvShape<128>::NW); }

// Varlen launches pass their tile lists (q_list: 128-row query tiles for dQ,
// kv_list: dK/dV key tiles) with their entry counts; the grids then run one
// work-group per (entry, head).
static int run_bwd(BwdParams base, int D, int dtype, int Hkv, int max_sq, int max_sk, int nbatch,
                   int causal, hipStream_t st, const int* q_list = nullptr, long long q_entries = 0,
                   const int* kv_list = nullptr, long long kv_entries = 0) {
  if (causal) base.wr = 0;
  if (q_entries > 0x7fffffffLL || kv_entries > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
  BwdParams kv = base;
  const int kv_keys = dkdv_keys(D);
  kv.tiles = kv_list;
  kv.n_tiles = kv_list ? (int)kv_entries : (max_sk + kv_keys - 1) / kv_keys;
  kv.n_heads = Hkv;
  kv.n_batch = kv_list ? 1 : nbatch;
  kv.reverse = 0;
  kv.balanced = causal ? 1 : 0;
  kv.group = kTileGroup;
  BwdParams dq = base;
  dq.tiles = q_list;
  dq.n_tiles = q_list ? (int)q_entries : (max_sq + 127) / 128;
  dq.n_heads = base.Hq;
  dq.n_batch = q_list ? 1 : nbatch;
  dq.reverse = causal ? 1 : 0;
  dq.balanced = causal ? 1 : 0;
  dq.group = kTileGroup;
  const long long nwg_kv = (long long)kv.n_tiles * kv.n_heads * kv.n_batch;
  const long long nwg_q = (long long)dq.n_tiles * dq.n_heads * dq.n_batch;
  if (nwg_kv > 0x7fffffffLL || nwg_q > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
  const bool sc = base.cap_log2 > 0.0f, al = base.alibi != nullptr;
  const bool bf = dtype == FA_DTYPE_BF16;
  const int nk = (int)nwg_kv, nq = (int)nwg_q;
  switch (D) {
    case 32:
      if (bf) launch_all<32, DT_BF16>(kv, dq, nk, nq, sc, al, st);
      else launch_all<32, DT_F16>(kv, dq, nk, nq, sc, al, st);
      break;
    case 64:
      if (bf) launch_all<64, DT_BF16>(kv, dq, nk, nq, sc, al, st);
      else launch_all<64, DT_F16>(kv, dq, nk, nq, sc, al, st);
      break;
    case 96:  // padded to 128 on chip
      if (bf) launch_all<128, DT_BF16, 96>(kv, dq, nk, nq, sc, al, st);
      else launch_all<128, DT_F16, 96>(kv, dq, nk, nq, sc, al, st);
      break;
    case 128:
      if (bf) launch_all<128, DT_BF16>(kv, dq, nk, nq, sc, al, st);
      else launch_all<128, DT_F16>(kv, dq, nk, nq, sc, al, st);
      break;
    default:
      if (bf) launch_all<256, DT_BF16>(kv, dq, nk, nq, sc, al, st);
      else launch_all<256, DT_F16>(kv, dq, nk, nq, sc, al, st);
      break;
  }
  return launch_status();
}

static void fill_common(BwdParams& p, const void* q, const void* k, const void* v, const void* out,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv, int Hq, int Hkv,
                        int D, float scale, int wl, int wr, float softcap, const float* alibi) {
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = (const uint16_t*)out;
  p.dout = (const uint16_t*)dout;
  p.lse = lse;
  p.dq = (uint16_t*)dq;
  p.dk = (uint16_t*)dk;
  p.dv = (uint16_t*)dv;
  p.Hq = Hq;
  p.g = Hq / Hkv;
  p.q_rstride = Hq * D;
  p.k_rstride = Hkv * D;
  p.o_rstride = Hq * D;
  p.dq_rstride = Hq * D;
  p.dkv_rstride = Hkv * D;
  p.scale = scale;
  p.scale_log2 = scale * kLog2e;
  p.scale_over_cap = softcap > 0.0f ? scale / softcap : 0.0f;
  p.cap_log2 = softcap * kLog2e;
  p.inv_cap_log2 = softcap > 0.0f ? 1.0f / (softcap * kLog2e) : 0.0f;
  p.alibi = alibi;
  p.wl = wl;
  p.wr = wr;
}

static bool bwd_ptrs_ok(const void* q, const void* k, const void* v, const void* out, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv, const float* alibi) {
  return aligned16(q) && aligned16(k) && aligned16(v) && aligned16(out) && aligned16(dout) &&
         aligned16(dq) && aligned16(dk) && aligned16(dv) && aligned4(lse) && (!alibi || aligned4(alibi));
}

}  // namespace fa

using namespace fa;

extern "C" size_t fa_bwd_workspace_size(int B, int Sq, int Sk, int Hq, int Hkv, int D, int deterministic) {
  (void)Sk;
  (void)Hkv;
  (void)D;
  (void)deterministic;
  if (B < 1 || Sq < 1 || Hq < 1) return 0;
  return 2 * align_up((size_t)B * Hq * Sq * sizeof(float), 256);
}

// Row-term arrays, then the query-tile list, then the key-tile list.
static size_t bwd_varlen_rows_bytes(int total_q, int Hq) {
  return align_up((size_t)total_q * Hq * sizeof(float), 256);
}

extern "C" size_t fa_bwd_varlen_workspace_size(int nseq, int total_q, int total_k, int Hq, int D,
                                               int deterministic) {
  (void)deterministic;
  if (nseq < 1 || total_q < 0 || total_k < 0 || Hq < 1) return 0;
  size_t n = 2 * bwd_varlen_rows_bytes(total_q, Hq);
  if (total_q > 0) n += varlen_list_bytes(total_q, nseq, 128);
  if (total_k > 0) n += varlen_list_bytes(total_k, nseq, dkdv_keys(D));
  return n;
}

// Row strides (elements between consecutive tokens) of q; k and v; dq;
// dk and dv; 0 = contiguous.  out and dout are always contiguous.
struct BwdStrides {
  int q, kv, dq, dkv;
};

static int bwd_dense(const void* q, const void* k, const void* v, const void* out, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv,
                     int B, int Sq, int Sk, int Hq, int Hkv, int D, int dtype,
                     float scale, int causal, int window_left, int window_right, float softcap,
                     const float* alibi_slopes, const DropSpec& drop, int deterministic,
                     void* workspace, size_t workspace_bytes, void* stream,
                     BwdStrides rs = BwdStrides{0, 0, 0, 0}) {
  int st = check_common(Hq, Hkv, D, dtype, scale, window_left, window_right, softcap);
  if (st) return st;
  if (B < 1 || Sq < 1 || Sk < 1) return FA_ERR_INVALID_ARG;
  if (!bwd_ptrs_ok(q, k, v, out, dout, lse, dq, dk, dv, alibi_slopes)) return FA_ERR_INVALID_ARG;
  const size_t need = fa_bwd_workspace_size(B, Sq, Sk, Hq, Hkv, D, deterministic);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return FA_ERR_WORKSPACE;
  BwdParams p{};
  fill_common(p, q, k, v, out, dout, lse, dq, dk, dv, Hq, Hkv, D, scale, window_left, window_right, softcap,
              alibi_slopes);
  p.dvec = (float*)workspace;
  p.lse2 = (float*)((char*)workspace + need / 2);
  p.Sq = Sq;
  p.Sk = Sk;
  p.drop = drop;
  if (rs.q) p.q_rstride = rs.q;
  if (rs.kv) p.k_rstride = rs.kv;
  if (rs.dq) p.dq_rstride = rs.dq;
  if (rs.dkv) p.dkv_rstride = rs.dkv;
  return run_bwd(p, D, dtype, Hkv, Sq, Sk, B, causal, (hipStream_t)stream);
}

static int bwd_varlen(const void* q, const void* k, const void* v, const void* out, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv,
                      const int* cu_seqlens_q, const int* cu_seqlens_k, int nseq,
                      int max_seqlen_q, int max_seqlen_k, int total_q, int total_k,
                      int Hq, int Hkv, int D, int dtype,
                      float scale, int causal, int window_left, int window_right, float softcap,
                      const float* alibi_slopes, const DropSpec& drop, int deterministic,
                      void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_common(Hq, Hkv, D, dtype, scale, window_left, window_right, softcap);
  if (st) return st;
  if (nseq < 1 || max_seqlen_q < 0 || max_seqlen_k < 0 || total_q < 0 || total_k < 0) return FA_ERR_INVALID_ARG;
  if (!aligned4(cu_seqlens_q) || !aligned4(cu_seqlens_k)) return FA_ERR_INVALID_ARG;
  // tensors of an empty side (no queries at all, or no keys at all) may be NULL
  const bool q_ok = total_q == 0 || (aligned16(q) && aligned16(out) && aligned16(dout) && aligned16(dq) &&
                                     aligned4(lse));
  const bool k_ok = total_k == 0 || (aligned16(k) && aligned16(v) && aligned16(dk) && aligned16(dv));
  if (!q_ok || !k_ok || (alibi_slopes && !aligned4(alibi_slopes))) return FA_ERR_INVALID_ARG;
  const size_t need = fa_bwd_varlen_workspace_size(nseq, total_q, total_k, Hq, D, deterministic);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace))) return FA_ERR_WORKSPACE;
  if (total_q == 0 && total_k == 0) return FA_OK;
  // With keys but no queries the dK/dV kernel still runs and writes dK = dV = 0
  // for every key row of a sequence; with queries but no keys the dQ kernel
  // writes dQ = 0.  Neither reads the tensors of the empty side.
  if (total_q == 0) max_seqlen_q = 0;
  if (total_k == 0) max_seqlen_k = 0;
  BwdParams p{};
  fill_common(p, q, k, v, out, dout, lse, dq, dk, dv, Hq, Hkv, D, scale, window_left, window_right, softcap,
              alibi_slopes);
  const size_t rows = bwd_varlen_rows_bytes(total_q, Hq);
  char* ws = (char*)workspace;
  p.dvec = (float*)ws;
  p.lse2 = (float*)(ws + rows);
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.total_q = total_q;
  p.drop = drop;
  // tile lists: query tiles heaviest (last) first for causal; key tiles of
  // a causal launch are heaviest first when taken from tile 0 up
  hipStream_t s = (hipStream_t)stream;
  int* q_list = nullptr;
  int* kv_list = nullptr;
  long long q_entries = 0, kv_entries = 0;
  char* lists = ws + 2 * rows;
  if (total_q > 0) {
    q_list = (int*)lists;
    q_entries = varlen_list_entries(total_q, nseq, 128);
    lists += varlen_list_bytes(total_q, nseq, 128);
    st = varlen_schedule(cu_seqlens_q, nseq, 128, (max_seqlen_q + 127) / 128, false, Hq, q_list, q_entries, s);
    if (st) return st;
  }
  if (total_k > 0) {
    const int kk = dkdv_keys(D);
    kv_list = (int*)lists;
    kv_entries = varlen_list_entries(total_k, nseq, kk);
    st = varlen_schedule(cu_seqlens_k, nseq, kk, (max_seqlen_k + kk - 1) / kk, causal != 0, Hkv, kv_list,
                         kv_entries, s);
    if (st) return st;
  }
  return run_bwd(p, D, dtype, Hkv, max_seqlen_q, max_seqlen_k, nseq, causal, s, q_list, q_entries, kv_list,
                 kv_entries);
}

extern "C" int fa_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv,
                      int B, int Sq, int Sk, int Hq, int Hkv, int D, int dtype,
                      float scale, int causal, int window_left, int window_right, float softcap,
                      const float* alibi_slopes, int deterministic,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_dense(q, k, v, out, dout, lse, dq, dk, dv, B, Sq, Sk, Hq, Hkv, D, dtype, scale, causal,
                   window_left, window_right, softcap, alibi_slopes, DropSpec{}, deterministic, workspace,
                   workspace_bytes, stream);
}

extern "C" int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* out, const void* dout,
                              const float* lse, void* dq, void* dk, void* dv,
                              int B, int Sq, int Sk, int Hq, int Hkv, int D, int dtype,
                              float scale, int causal, int window_left, int window_right, float softcap,
                              const float* alibi_slopes, float dropout_p, unsigned long long seed,
                              unsigned long long offset, int deterministic,
                              void* workspace, size_t workspace_bytes, void* stream) {
  DropSpec drop;
  if (!make_drop(dropout_p, seed, offset, drop)) return FA_ERR_INVALID_ARG;
  return bwd_dense(q, k, v, out, dout, lse, dq, dk, dv, B, Sq, Sk, Hq, Hkv, D, dtype, scale, causal,
                   window_left, window_right, softcap, alibi_slopes, drop, deterministic, workspace,
                   workspace_bytes, stream);
}

extern "C" int fa_bwd_qkvpacked(const void* qkv, const void* out, const void* dout, const float* lse,
                                void* dqkv, int B, int S, int H, int D, int dtype,
                                float scale, int causal, int window_left, int window_right, float softcap,
                                const float* alibi_slopes, int deterministic,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (!aligned16(qkv) || !aligned16(dqkv) || H < 1 || D < 1) return FA_ERR_INVALID_ARG;
  const uint16_t* b = (const uint16_t*)qkv;
  uint16_t* g = (uint16_t*)dqkv;
  const int hd = H * D;
  return bwd_dense(b, b + hd, b + 2 * hd, out, dout, lse, g, g + hd, g + 2 * hd, B, S, S, H, H, D, dtype,
                   scale, causal, window_left, window_right, softcap, alibi_slopes, DropSpec{}, deterministic,
                   workspace, workspace_bytes, stream, BwdStrides{3 * hd, 3 * hd, 3 * hd, 3 * hd});
}

extern "C" int fa_bwd_kvpacked(const void* q, const void* kv, const void* out, const void* dout,
                               const float* lse, void* dq, void* dkv,
                               int B, int Sq, int Sk, int Hq, int Hkv, int D, int dtype,
                               float scale, int causal, int window_left, int window_right, float softcap,
                               const float* alibi_slopes, int deterministic,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (!aligned16(kv) || !aligned16(dkv) || Hkv < 1 || D < 1) return FA_ERR_INVALID_ARG;
  const uint16_t* b = (const uint16_t*)kv;
  uint16_t* g = (uint16_t*)dkv;
  const int hd = Hkv * D;
  return bwd_dense(q, b, b + hd, out, dout, lse, dq, g, g + hd, B, Sq, Sk, Hq, Hkv, D, dtype, scale, causal,
                   window_left, window_right, softcap, alibi_slopes, DropSpec{}, deterministic, workspace,
                   workspace_bytes, stream, BwdStrides{0, 2 * hd, 0, 2 * hd});
}

extern "C" int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* out, const void* dout,
                             const float* lse, void* dq, void* dk, void* dv,
                             const int* cu_seqlens_q, const int* cu_seqlens_k, int nseq,
                             int max_seqlen_q, int max_seqlen_k, int total_q, int total_k,
                             int Hq, int Hkv, int D, int dtype,
                             float scale, int causal, int window_left, int window_right, float softcap,
                             const float* alibi_slopes, int deterministic,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_varlen(q, k, v, out, dout, lse, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, nseq, max_seqlen_q,
                    max_seqlen_k, total_q, total_k, Hq, Hkv, D, dtype, scale, causal, window_left,
                    window_right, softcap, alibi_slopes, DropSpec{}, deterministic, workspace,
                    workspace_bytes, stream);
}

extern "C" int fa_bwd_varlen_dropout(const void* q, const void* k, const void* v, const void* out,
                                     const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                     const int* cu_seqlens_q, const int* cu_seqlens_k, int nseq,
                                     int max_seqlen_q, int max_seqlen_k, int total_q, int total_k,
                                     int Hq, int Hkv, int D, int dtype,
                                     float scale, int causal, int window_left, int window_right,
                                     float softcap, const float* alibi_slopes, float dropout_p,
                                     unsigned long long seed, unsigned long long offset, int deterministic,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  DropSpec drop;
  if (!make_drop(dropout_p, seed, offset, drop)) return FA_ERR_INVALID_ARG;
  return bwd_varlen(q, k, v, out, dout, lse, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, nseq, max_seqlen_q,
                    max_seqlen_k, total_q, total_k, Hq, Hkv, D, dtype, scale, causal, window_left,
                    window_right, softcap, alibi_slopes, drop, deterministic, workspace, workspace_bytes,
                    stream);
}
