// fa_fwd.hip — forward pass of exact tiled attention on gfx950.
//
// Method (page "FlashAttention 实战指南：如何把训练内存省 20 倍、速度提 4 倍", section
// "FlashAttention 的做法是三个手段配合"): Q, K, V are cut into blocks, the current
// block is staged on chip, QK^T and the softmax of that block are done there,
// and an online softmax updates a running row maximum and row sum block by
// block, so the n x n matrix never exists in memory.
//
// Work decomposition (one work-group = 4 waves = 128 query rows of one head):
//   * each wave owns 32 query rows; their Q fragment stays in VGPRs for the
//     whole key loop (B operand of S^T = K Q^T);
//   * K and V tiles of 64 keys are copied HBM -> LDS by DMA
//     (global_load_lds) into separate double buffers; the copies of K for
//     tile t+2 and V for tile t+1 overlap the work on tile t;
//   * the key loop is software pipelined: the MFMAs of S for tile t+1 are
//     issued in the same basic block as the exponentials of tile t, so one
//     wave keeps the matrix core busy while its VALU does the softmax;
//   * S^T = K Q^T on MFMA 32x32x16 puts one query per lane (two lanes per
//     query, 16 keys each), so the row max needs one cross-lane step and the
//     row sum none until the epilogue;
//   * O^T += V^T P^T: P^T is fed back from the S^T accumulator registers in
//     acc-order and V^T is read from the row-major V tile with transposing
//     LDS reads;
//   * the online softmax works in the log2 domain: p = exp2(x - m).
#include "fa_device.h"
#include "fa_host.h"

namespace fa {

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const int* cu_q;  // packed layout when non-null
  const int* cu_k;
  int Sq, Sk;       // per-batch lengths (dense layout)
  int Hq, g;        // query heads, query heads per K/V head
  int total_q;      // packed layout: LSE row stride
  int q_rstride;    // elements between consecutive tokens of q (Hq * D unless packed)
  int k_rstride;    // elements between consecutive tokens of k and of v (Hkv * D unless packed)
  int o_rstride;    // elements between consecutive tokens of o (Hq * D)
  float scale_log2;     // scale * log2(e)
  float scale_over_cap; // scale / softcap
  float cap_log2;       // softcap * log2(e)
  const float* alibi;
  int wl, wr;           // window, causal folded into wr = 0
  int n_qtiles, n_heads, n_batch;
  int reverse;          // causal: heaviest tiles first
  int group;            // causal: pairs per XCD group (tile_id)
  const int* tiles;     // varlen tile list (entries x 2 ints), or NULL
  DropSpec drop;        // DROP kernels only
  // FP8 kernels: q and k are OCP e4m3 bytes, v the bfloat16 copy of the fp8
  // values; per-(batch, K/V head) dequantisation factors, NULL = 1
  const float* dsc_q;
  const float* dsc_k;
  const float* dsc_v;
};

// D = 256 needs the whole register file of a SIMD (Q fragment 64, O
// accumulator 128, two S tiles 64) and 128 KB of LDS: one wave per SIMD.
// FP8: S = K Q^T runs on the fp8 matrix instruction (32 x 32 x 64) from
// fp8 Q fragments and fp8 K tiles; P V stays in bfloat16 (V converted
// exactly beforehand), so only the logits change precision and they are
// exact products of the fp8 inputs.
// DG < D: the head dim in memory is DG and is padded to D on chip (zero Q
// columns and zero K/V tile columns, so S and the first DG columns of O are
// exact; the rest is never stored).
template <int D, int DT, bool SOFTCAP, bool ALIBI, bool DROP, bool FP8 = false, int DG = D>
__global__ __launch_bounds__(256, D >= 256 ? 1 : 2) void fwd_kernel(FwdParams p) {
  constexpr int BR = 128, BC = 64;
  constexpr int KC = D / 16;               // MFMA steps along D
  constexpr int DB = D / 32;               // 32-wide output blocks along D
  constexpr int TILE = BC * D * 2;         // bytes of one K or V tile
  __shared__ __attribute__((aligned(1024))) char kb0[TILE];
  __shared__ __attribute__((aligned(1024))) char kb1[TILE];
  __shared__ __attribute__((aligned(1024))) char vb0[TILE];
  __shared__ __attribute__((aligned(1024))) char vb1[TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, known uniform
  const int g = lane >> 5, r = lane & 31;
  const uint32_t nb = nat_base<D>(lane);
  const uint32_t tb = tr_base<D>(lane);

  // logical tile id -> (q tile, head, batch)
  // causal: the last query tiles see the most keys
  TileId tid3;
  if (p.tiles) {
    if (!tile_from_list(p.tiles, p.n_heads, tid3)) return;  // unused list entry
  } else {
    tid3 = tile_id(p.n_qtiles, p.n_heads, p.n_batch, p.reverse != 0, p.reverse != 0, p.group);
  }
  const int tq = tid3.t, h = tid3.h, b = tid3.b;

  int q_start, Sq, k_start, Sk;
  if (p.cu_q) {
    q_start = p.cu_q[b];
    Sq = p.cu_q[b + 1] - q_start;
    k_start = p.cu_k[b];
    Sk = p.cu_k[b + 1] - k_start;
  } else {
    q_start = b * p.Sq;
    Sq = p.Sq;
    k_start = b * p.Sk;
    Sk = p.Sk;
  }
  const int q0 = tq * BR;
  if (q0 >= Sq) return;  // uniform over the work-group
  const int hk = h / p.g;
  const int off = Sk - Sq;
  const MaskSpec mask{p.wl, p.wr};

  const uint16_t* qbase = p.q + (int64_t)q_start * p.q_rstride + h * DG;
  const uint16_t* kbase = p.k + (int64_t)k_start * p.k_rstride + hk * DG;
  const uint16_t* vbase = p.v + (int64_t)k_start * p.k_rstride + hk * DG;

  const int qend = min(q0 + BR, Sq);
  int kv_lo = 0, kv_hi = Sk;
  if (p.wl >= 0) kv_lo = max(0, q0 + off - p.wl);
  if (p.wr >= 0) kv_hi = min(Sk, qend - 1 + off + p.wr + 1);

  const int wrow0 = q0 + 32 * w;
  const int wrow1 = min(wrow0 + 31, Sq - 1);
  const int my_row = wrow0 + r;
  const bool row_ok = my_row < Sq;
  const int ip = my_row + off;

  u32x4 qreg[KC];
  i32x8 q8[D / 64 > 0 ? D / 64 : 1];
  if constexpr (FP8) {
    // byte j of step c, half g = element 64 c + 32 g + j of the fp8 row
    const uint8_t* qrow8 = reinterpret_cast<const uint8_t*>(p.q) + ((int64_t)q_start + my_row) * p.q_rstride + h * D;
#pragma unroll
    for (int c = 0; c < D / 64; ++c) {
      const u32x4 lo = row_ok ? gload128(qrow8 + 64 * c + 32 * g) : u32x4{0, 0, 0, 0};
      const u32x4 hi = row_ok ? gload128(qrow8 + 64 * c + 32 * g + 16) : u32x4{0, 0, 0, 0};
      q8[c] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
  } else {
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const bool in = DG == D || (2 * c + g) * 8 < DG;
      qreg[c] = (row_ok && in) ? gload128(qbase + (int64_t)my_row * p.q_rstride + (2 * c + g) * 8)
                               : u32x4{0, 0, 0, 0};
    }
  }
  // FP8: the logits are scaled by the dequantisation factors of q and k
  float dqk = 1.0f, dsv = 1.0f;
  if constexpr (FP8) {
    const int64_t di = (int64_t)b * (p.Hq / p.g) + hk;
    dqk = (p.dsc_q ? p.dsc_q[di] : 1.0f) * (p.dsc_k ? p.dsc_k[di] : 1.0f);
    dsv = p.dsc_v ? p.dsc_v[di] : 1.0f;
  }
  const float sl2 = p.scale_log2 * dqk, soc = p.scale_over_cap * dqk;

  f32x16 oacc[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) oacc[d] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;
  const float fs = (SOFTCAP || ALIBI) ? 1.0f : sl2;
  const float slope_log2 = ALIBI ? p.alibi[h] * kLog2e : 0.0f;
  const uint32_t bh = (uint32_t)(b * p.Hq + h);  // dropout counter word 2

  if (kv_lo < kv_hi) {
    const int t_lo = kv_lo / BC, t_hi = (kv_hi + BC - 1) / BC;
    auto dma_k = [&](int t, char* dst) {
      if constexpr (FP8) {
        // fp8 rows of D bytes copied as D / 2 16-bit elements
        const uint16_t* kb8 = reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(p.k) +
                                                                (int64_t)k_start * p.k_rstride + hk * D);
        dma_tile<(D >= 64 ? D / 2 : 32), BC, 4>(dst, kb8, p.k_rstride / 2, t * BC, Sk, w, lane);
      } else {
        dma_tile<D, BC, 4, true, DG>(dst, kbase, p.k_rstride, t * BC, Sk, w, lane);
      }
    };
    auto dma_v = [&](int t, char* dst) {
      dma_tile<D, BC, 4, true, DG>(dst, vbase, p.k_rstride, t * BC, Sk, w, lane);
    };

    // S^T = K Q^T for the 64 keys of LDS tile `kt` (raw dot products).
    auto qk = [&](const char* kt, uint32_t nbv, f32x16 (&sa)[2]) {
      if constexpr (FP8) {
        // A operand: key row lane % 32, bytes 64 c + 32 g .. + 31 (chunks
        // 4c + 2g and 4c + 2g + 1 of the D-byte row, swizzled like a
        // D/2-element 16-bit row)
        constexpr int DH = D >= 64 ? D / 2 : 32;
        const uint32_t nb8 = opaque(row_base<DH>(lane & 31) ^ ((uint32_t)(2 * g) << 4));
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          sa[kb] = f32x16{};
#pragma unroll
          for (int c = 0; c < D / 64; ++c) {
            const char* t8 = kt + (kb * 32) * D;
            const u32x4 lo = lds_read128(t8, nb8 ^ ((uint32_t)c << 6));
            const u32x4 hi = lds_read128(t8, nb8 ^ ((uint32_t)c << 6) ^ 16u);
            const i32x8 ka = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                              (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            sa[kb] = mfma32_fp8(ka, q8[c], sa[kb]);
          }
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          sa[kb] = f32x16{};
#pragma unroll
          for (int c = 0; c < KC; ++c) {
            sa[kb] = mfma32<DT>(lds_nat(kt + (kb * 32) * (D * 2), nbv, c), qreg[c], sa[kb]);
          }
        }
      }
    };

    // Logits of tile t in the log2 domain (up to the folded scale fs), masked
    // entries at -inf (keys past Sk hold a copy of the last key).
    auto logits = [&](int t, f32x16 (&sa)[2]) {
      const int j0 = t * BC;
      if constexpr (SOFTCAP || ALIBI) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float x = sa[kb][i];
            const int j = j0 + 32 * kb + frag_row(i, g);
            if constexpr (SOFTCAP) x = p.cap_log2 * tanh_exp(x * soc);
            else x = x * sl2;
            if constexpr (ALIBI) x -= slope_log2 * (float)abs(ip - j);
            sa[kb][i] = x;
          }
        }
      }
      const int cls = (wrow0 < Sq) ? classify(wrow0 + off, wrow1 + off, j0, j0 + BC - 1, Sk, mask) : 0;
      if (cls != 2) {
        const LaneRange kr = keys_for_row(row_ok, ip, Sk, mask);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const RangeTest rt = range_test(kr, j0 + 32 * kb + 4 * g);
#pragma unroll
          for (int i = 0; i < 16; ++i) sa[kb][i] = in_range(rt, i) ? sa[kb][i] : -INFINITY;
        }
      }
    };

    // Lazy online-softmax update of the exponent reference from this lane's
    // tile maximum mx (before the lane-half exchange and the folded scale).
    // The reference m_run moves only when the tile max exceeds it by more
    // than kRescaleSlack; until then p <= 2^kRescaleSlack, which the float32
    // sums and the 16-bit P operand carry without loss, and the rescale of O
    // (64 multiplies per lane) is skipped.  Returns m_use.
    auto rescale = [&](float mx) -> float {
      mx = pair_max32(mx) * fs;
      if (__any(mx > m_run + kRescaleSlack)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2(m_run - m_new);
#pragma unroll
        for (int d = 0; d < DB; ++d) oacc[d] *= alpha;
        l_run *= alpha;
        m_run = m_new;
      }
      return (m_run == -INFINITY) ? 0.0f : m_run;
    };

    auto prep = [&](int t, f32x16 (&sa)[2]) -> float {
      logits(t, sa);
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sa[kb][i]);
      return rescale(mx);
    };

    // Dropout keep words of tile t (two 32-key halves).
    auto keepw = [&](int t, uint32_t (&kw)[2][4]) {
      if constexpr (DROP) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) drop_words<false>(p.drop, bh, my_row, t * BC + 32 * kb, lane, kw[kb]);
      }
    };

    // P = 2^(x - m) as four 16-bit B operands (acc-order), row sums of the
    // float32 weights into l_run (dropped weights count in the sum and enter
    // the product as 0).
    auto expo = [&](f32x16 (&sa)[2], float m_use, const uint32_t (&kw)[2][4], u32x4 (&pb)[4]) {
      float lsum = 0.0f, lsum2 = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pv = fast_exp2(fmaf(sa[kb][i], fs, -m_use));
          if (i & 1) lsum2 += pv;
          else lsum += pv;
          sa[kb][i] = (DROP && !drop_keep(kw[kb], i, p.drop.t)) ? 0.0f : pv;
        }
      l_run += lsum + lsum2;
#pragma unroll
      for (int mk = 0; mk < 4; ++mk) pb[mk] = pack_frag_half<DT>(sa[mk >> 1], mk & 1);
    };

    // O^T += V^T P^T over the 64 keys of LDS tile `vt`.
    auto pv = [&](const char* vt, uint32_t tbv, const u32x4 (&pb)[4]) {
#pragma unroll
      for (int mk = 0; mk < 4; ++mk) {
#pragma unroll
        for (int d = 0; d < DB; ++d) {
          oacc[d] = mfma32<DT>(lds_At<D>(vt + (16 * mk) * (D * 2), tbv, d), pb[mk], oacc[d]);
        }
      }
    };

    // First four K fragments of the next S (LDS tile `kn`).  A step issues
    // them before its softmax prologue, so their LDS latency is hidden by it.
    auto k_ring = [&](const char* kn, uint32_t nbv, u32x4 (&kr)[4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i) kr[i] = lds_nat(kn + (i / KC) * 32 * (D * 2), nbv, i % KC);
    };

    // The pipelined block in an explicit instruction order.  S of the next
    // tile: a ring of four K fragments keeps four LDS reads in flight ahead of
    // the MFMA that consumes them; the first MXS MFMAs carry the current
    // tile's maximum and the exponent-reference update, each later one a
    // slice of the current tile's exponentials; once the K ring has nothing left to fetch,
    // its last slots start the first three V^T fragments.  Then O += P V with
    // a ring of three V^T fragments (six transposed reads) in flight, with
    // the packing of P and the row sum spread over those MFMAs, so the
    // element-wise work is split between both halves of the step.  (Dropout
    // tiles run the plain loop, never this block.)  sched_barrier fences keep the scheduler
    // from pulling each read down next to its MFMA, which would expose the
    // whole LDS latency on every MFMA.
    auto fused = [&](const char* kn, const char* vt, uint32_t nbv, uint32_t tbv, u32x4 (&kr)[4],
                     f32x16 (&sc)[2], f32x16 (&sn)[2]) {
      constexpr int NS = 2 * KC;    // S MFMAs per tile
      constexpr int MXS = 2;        // S MFMAs that carry the tile maximum
      constexpr int NP = 4 * DB;    // P V MFMAs per tile
      constexpr int LEAD = DB >= 2 ? 2 : 1;
      sn[0] = f32x16{};
      sn[1] = f32x16{};
      float lsum = 0.0f, lsum2 = 0.0f;
      float mx = -INFINITY, m_use = 0.0f;
      u32x4 pb[4];
      u32x4 vr[3];
      bool pb0 = false;
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int kb = i / KC, c = i % KC;
        sn[kb] = mfma32<DT>(kr[i & 3], qreg[c], sn[kb]);
        if (i + 4 < NS) {
          kr[i & 3] = lds_nat(kn + ((i + 4) / KC) * 32 * (D * 2), nbv, (i + 4) % KC);
        } else if (i + 4 - NS < 3) {
          const int j = i + 4 - NS;
          vr[j] = lds_At<D>(vt + (16 * (j / DB)) * (D * 2), tbv, j % DB);
        }
        if (i < MXS) {
          // the tile maximum of the current tile, under the first S MFMAs of
          // the next one (they do not depend on it)
#pragma unroll
          for (int e = 32 * i / MXS; e < 32 * (i + 1) / MXS; ++e) mx = fmaxf(mx, sc[e >> 4][e & 15]);
        } else {
          if (i == MXS) m_use = rescale(mx);
          // the current tile's exponentials, spread over the remaining S MFMAs
#pragma unroll
          for (int e = 32 * (i - MXS) / (NS - MXS); e < 32 * (i - MXS + 1) / (NS - MXS); ++e)
            sc[e >> 4][e & 15] = fast_exp2(fmaf(sc[e >> 4][e & 15], fs, -m_use));
          // the first P operand is packed once its eight weights exist; the
          // other three, and the row sum, go under the P V MFMAs
          if (!pb0 && 32 * (i - MXS + 1) / (NS - MXS) >= 8) {
            pb[0] = pack_frag_half<DT>(sc[0], 0);
            pb0 = true;
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int mk = i / DB, d = i % DB;
        oacc[d] = mfma32<DT>(vr[i % 3], pb[mk], oacc[d]);
        if (i + 3 < NP) vr[i % 3] = lds_At<D>(vt + (16 * ((i + 3) / DB)) * (D * 2), tbv, (i + 3) % DB);
        // P operand mn (used from MFMA mn * DB on) is packed LEAD MFMAs ahead
#pragma unroll
        for (int mn = 1; mn < 4; ++mn)
          if (i == mn * DB - LEAD) pb[mn] = pack_frag_half<DT>(sc[mn >> 1], mn & 1);
        // row sum of the float32 weights (the LSE needs their exact sum, not
        // that of the 16-bit P operand), two chains
#pragma unroll
        for (int e = i * 32 / NP; e < (i + 1) * 32 / NP; ++e) {
          if (e & 1) lsum2 += sc[e >> 4][e & 15];
          else lsum += sc[e >> 4][e & 15];
        }
        // pin the partial sums here (an empty asm that reads and redefines
        // them), so they run under this MFMA instead of being sunk after the
        // block as one serial chain
        asm volatile("" : "+v"(lsum), "+v"(lsum2));
        __builtin_amdgcn_sched_barrier(0);
      }
      l_run += lsum + lsum2;
    };

    // Pipelined step for tile t (t + 1 < t_hi): `sc` holds S of tile t, the
    // MFMAs of S for tile t + 1 (K in `kn`, into `sn`) run in the same basic
    // block as the exponentials of tile t, then O += P V with V of tile t in
    // `vt`.  DMA: K of tile t + 2 into `kdst` (K of tile t, already used),
    // V of tile t + 1 into `vdst` (V of tile t - 1, already used).
    auto step = [&](int t, const char* kn, const char* vt, char* kdst, char* vdst, f32x16 (&sc)[2],
                    f32x16 (&sn)[2]) {
      if (t + 2 < t_hi) dma_k(t + 2, kdst);
      dma_v(t + 1, vdst);
      const uint32_t nbv = opaque(nb), tbv = opaque(tb);
      u32x4 kr[4];
      k_ring(kn, nbv, kr);
      logits(t, sc);
      fused(kn, vt, nbv, tbv, kr, sc, sn);
      dma_wait();
      __syncthreads();
    };

    // Final tile: no next S, no DMA.
    auto last = [&](int t, const char* vt, f32x16 (&sc)[2]) {
      const uint32_t tbv = opaque(tb);
      uint32_t kw[2][4];
      keepw(t, kw);
      const float m_use = prep(t, sc);
      u32x4 pb[4];
      expo(sc, m_use, kw, pb);
      pv(vt, tbv, pb);
    };

    // Four distinct LDS arrays: K and V, double buffered, so reads of one are
    // never ordered behind the DMA into another.
    f32x16 sA[2], sB[2];
    zero_pad<D, BC, DG>(kb0, tid, 256);
    zero_pad<D, BC, DG>(kb1, tid, 256);
    zero_pad<D, BC, DG>(vb0, tid, 256);
    zero_pad<D, BC, DG>(vb1, tid, 256);
    if constexpr (DROP || D >= 256 || FP8) {
      // With dropout the generator's integer work dominates the VALU, and at
      // D = 256 two S tiles next to the O accumulator exceed the register
      // file, so the tiles run one after another (S, softmax, P V) with the
      // next tile's K and V copied in underneath.
      auto plain = [&](int t, const char* kt, const char* vt, char* kdst, char* vdst) {
        if (t + 1 < t_hi) {
          dma_k(t + 1, kdst);
          dma_v(t + 1, vdst);
        }
        qk(kt, opaque(nb), sA);
        last(t, vt, sA);
        dma_wait();
        __syncthreads();
      };
      dma_k(t_lo, kb0);
      dma_v(t_lo, vb0);
      dma_wait();
      __syncthreads();
      int t = t_lo;
      for (; t + 1 < t_hi; t += 2) {
        plain(t, kb0, vb0, kb1, vb1);
        plain(t + 1, kb1, vb1, kb0, vb0);
      }
      if (t < t_hi) plain(t, kb0, vb0, kb1, vb1);
    } else {
    dma_k(t_lo, kb0);
    dma_v(t_lo, vb0);
    if (t_lo + 1 < t_hi) dma_k(t_lo + 1, kb1);
    dma_wait();
    __syncthreads();
    qk(kb0, nb, sA);
    __syncthreads();  // every wave is done with kb0 before it is refilled
    int t = t_lo;
    for (; t + 2 < t_hi; t += 2) {
      step(t, kb1, vb0, kb0, vb1, sA, sB);
      step(t + 1, kb0, vb1, kb1, vb0, sB, sA);
    }
    if (t + 1 < t_hi) {
      step(t, kb1, vb0, kb0, vb1, sA, sB);
      last(t + 1, vb1, sB);
    } else {
      last(t, vb0, sA);
    }
    }
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 ----
  const float l_tot = pair_sum32(l_run);
  if (row_ok) {
    const float inv = l_tot > 0.0f ? (DROP ? p.drop.scale : 1.0f) * (FP8 ? dsv : 1.0f) / l_tot : 0.0f;
    uint16_t* orow = p.o + (int64_t)(q_start + my_row) * p.o_rstride + h * DG;
#pragma unroll
    for (int d = 0; d < DB; ++d) {
      if (32 * d >= DG) continue;  // padded columns
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        u32x2 v2;
        v2[0] = pack2<DT>(oacc[d][4 * qd + 0] * inv, oacc[d][4 * qd + 1] * inv);
        v2[1] = pack2<DT>(oacc[d][4 * qd + 2] * inv, oacc[d][4 * qd + 3] * inv);
        gstore64(orow + 32 * d + 8 * qd + 4 * g, v2);
      }
    }
    if (p.lse && g == 0) {
      const float L = l_tot > 0.0f ? (m_run + fast_log2(l_tot)) * kLn2 : INFINITY;
      const int64_t li = p.cu_q ? (int64_t)h * p.total_q + q_start + my_row
                                : ((int64_t)b * p.Hq + h) * Sq + my_row;
      p.lse[li] = L;
    }
  }
}

template <int D, int DT, bool DROP, int DG = D>
static void launch_fwd_dt(const FwdParams& prm, bool softcap, bool alibi, int nwg, hipStream_t st) {
  dim3 grid(nwg), block(256);
  if (softcap) {
    if (alibi) hipLaunchKernelGGL((fwd_kernel<D, DT, true, true, DROP, false, DG>), grid, block, 0, st, prm);
    else hipLaunchKernelGGL((fwd_kernel<D, DT, true, false, DROP, false, DG>), grid, block, 0, st, prm);
  } else {
    if (alibi) hipLaunchKernelGGL((fwd_kernel<D, DT, false, true, DROP, false, DG>), grid, block, 0, st, prm);
    else hipLaunchKernelGGL((fwd_kernel<D, DT, false, false, DROP, false, DG>), grid, block, 0, st, prm);
  }
}

template <int D>
static void launch_fwd_fp8(const FwdParams& prm, bool softcap, bool alibi, int nwg, hipStream_t st) {
  dim3 grid(nwg), block(256);
  if (softcap) {
    if (alibi) hipLaunchKernelGGL((fwd_kernel<D, DT_BF16, true, true, false, true>), grid, block, 0, st, prm);
    else hipLaunchKernelGGL((fwd_kernel<D, DT_BF16, true, false, false, true>), grid, block, 0, st, prm);
  } else {
    if (alibi) hipLaunchKernelGGL((fwd_kernel<D, DT_BF16, false, true, false, true>), grid, block, 0, st, prm);
    else hipLaunchKernelGGL((fwd_kernel<D, DT_BF16, false, false, false, true>), grid, block, 0, st, prm);
  }
}

// fp8 (OCP e4m3) -> bfloat16, 16 bytes per thread; exact, since every e4m3
// value is a bfloat16 value.
__global__ __launch_bounds__(256) void fp8_to_bf16_kernel(const uint8_t* src, uint16_t* dst, int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n16) return;
  const u32x4 v = gload128(src + 16 * i);
  uint32_t o[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[e], false);  // bytes 0, 1
    const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[e], true);   // bytes 2, 3
    o[2 * e] = pack2<DT_BF16>(a[0], a[1]);
    o[2 * e + 1] = pack2<DT_BF16>(b[0], b[1]);
  }
  gstore128(dst + 16 * i, u32x4{o[0], o[1], o[2], o[3]});
  gstore128(dst + 16 * i + 8, u32x4{o[4], o[5], o[6], o[7]});
}

template <int D, int DT, int DG = D>
static void launch_fwd_d(const FwdParams& prm, bool softcap, bool alibi, bool drop, int nwg, hipStream_t st) {
  if (drop) launch_fwd_dt<D, DT, true, DG>(prm, softcap, alibi, nwg, st);
  else launch_fwd_dt<D, DT, false, DG>(prm, softcap, alibi, nwg, st);
}

static int run_fwd(FwdParams& prm, int D, int dtype, float scale, float softcap, int causal,
                   int max_sq, int nbatch, hipStream_t st, bool fp8 = false, long long list_entries = 0) {
  prm.scale_log2 = scale * kLog2e;
  prm.scale_over_cap = softcap > 0.0f ? scale / softcap : 0.0f;
  prm.cap_log2 = softcap * kLog2e;
  if (causal) prm.wr = 0;
  prm.n_heads = prm.Hq;
  if (prm.tiles) {
    if (list_entries > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
    prm.n_qtiles = (int)list_entries;
    prm.n_batch = 1;
  } else {
    prm.n_qtiles = (max_sq + 127) / 128;
    prm.n_batch = nbatch;
  }
  prm.reverse = causal ? 1 : 0;
  prm.group = kTileGroup;
  // a varlen tile list replaces the (tile, head, sequence) grid: n_qtiles
  // then counts list entries and n_batch is 1
  const long long nwg = (long long)prm.n_qtiles * prm.n_heads * prm.n_batch;
  if (nwg <= 0) return FA_OK;
  if (nwg > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
  const bool sc = softcap > 0.0f, al = prm.alibi != nullptr, dr = prm.drop.t > 0;
  prof_before(FA_KERNEL_FWD, st);
  const bool bf = dtype == FA_DTYPE_BF16;
  if (fp8) {
    if (D == 128) launch_fwd_fp8<128>(prm, sc, al, (int)nwg, st);
    else launch_fwd_fp8<64>(prm, sc, al, (int)nwg, st);
    prof_after(FA_KERNEL_FWD, st);
    return launch_status();
  }
  switch (D) {
    case 32:
      if (bf) launch_fwd_d<32, DT_BF16>(prm, sc, al, dr, (int)nwg, st);
      else launch_fwd_d<32, DT_F16>(prm, sc, al, dr, (int)nwg, st);
      break;
    case 64:
      if (bf) launch_fwd_d<64, DT_BF16>(prm, sc, al, dr, (int)nwg, st);
      else launch_fwd_d<64, DT_F16>(prm, sc, al, dr, (int)nwg, st);
      break;
    case 96:  // padded to 128 on chip
      if (bf) launch_fwd_d<128, DT_BF16, 96>(prm, sc, al, dr, (int)nwg, st);
      else launch_fwd_d<128, DT_F16, 96>(prm, sc, al, dr, (int)nwg, st);
      break;
    case 128:
      if (bf) launch_fwd_d<128, DT_BF16>(prm, sc, al, dr, (int)nwg, st);
      else launch_fwd_d<128, DT_F16>(prm, sc, al, dr, (int)nwg, st);
      break;
    default:
      if (bf) launch_fwd_d<256, DT_BF16>(prm, sc, al, dr, (int)nwg, st);
      else launch_fwd_d<256, DT_F16>(prm, sc, al, dr, (int)nwg, st);
      break;
  }
  prof_after(FA_KERNEL_FWD, st);
  return launch_status();
}

// ------------------------------------------------------ varlen tile list --
// Level-major list (more than kListSortMax sequences).  One work-group of
// 1024 threads writes the list (layout and order in
// fa_host.h).  Levels are taken in passes of TP <= 1024; in a pass, thread
// (lvl, c) owns level lvl and the c-th of 1024 / TP contiguous chunks of the
// sequences: it counts the chunk's sequences with a tile at that level,
// chunk counts and level totals give every (level, chunk) its first slot,
// and it then writes the chunk's entries in sequence order.  Integer work
// only; the list is the same on every call.
__global__ __launch_bounds__(1024) void varlen_schedule_kernel(const int* cu, int nseq, int tile, int levels,
                                                              int ascending, int* list, int n_entries) {
  __shared__ int cnt[1024];
  __shared__ int ltot[1024];
  __shared__ int lstart[1024];
  __shared__ int sbase;
  const int tid = threadIdx.x;
  const int TP = levels < 1024 ? (levels > 0 ? levels : 1) : 1024;
  const int C = 1024 / TP;
  const int lvl = tid % TP, c = tid / TP;
  const bool active = c < C;
  const int CS = (nseq + C - 1) / C;
  const int s0 = min(nseq, c * CS), s1 = min(nseq, s0 + CS);
  auto ntiles = [&](int sq) {
    const int len = cu[sq + 1] - cu[sq];
    return len > 0 ? (len + tile - 1) / tile : 0;
  };
  int base = 0;
  for (int L0 = 0; L0 < levels; L0 += TP) {
    const int npass = min(TP, levels - L0);
    const int k = L0 + lvl;
    const int t = ascending ? k : levels - 1 - k;
    const bool mine = active && lvl < npass;
    int n = 0;
    if (mine)
      for (int sq = s0; sq < s1; ++sq) n += ntiles(sq) > t;
    if (active) cnt[tid] = n;
    __syncthreads();
    if (tid < npass) {
      int tt = 0;
      for (int cc = 0; cc < C; ++cc) tt += cnt[cc * TP + tid];
      ltot[tid] = tt;
    }
    __syncthreads();
    if (tid == 0) {
      int acc = base;
      for (int l = 0; l < npass; ++l) {
        lstart[l] = acc;
        acc += ltot[l];
      }
      sbase = acc;
    }
    __syncthreads();
    if (mine) {
      int pos = lstart[lvl];
      for (int cc = 0; cc < c; ++cc) pos += cnt[cc * TP + lvl];
      for (int sq = s0; sq < s1; ++sq) {
        if (ntiles(sq) > t) {
          list[2 * pos] = sq;
          list[2 * pos + 1] = t;
          ++pos;
        }
      }
    }
    base = sbase;
    __syncthreads();  // cnt and lstart are rewritten by the next pass
  }
  for (int e = base + tid; e < n_entries; e += 1024) {
    list[2 * e] = -1;
    list[2 * e + 1] = -1;
  }
}

// Grouped list (nseq <= kListSortMax).  One work-group of 1024 threads:
//  1. sorts the sequences by tile count, most first (ties: lower index
//     first), with a bitonic sort of (count, index) keys in LDS;
//  2. cuts the sorted order into groups of `group` sequences and gives each
//     group its first slot (prefix sum of the groups' tile counts);
//  3. writes each group level by level: entry (sorted rank r, tile t) goes
//     to the group's first slot + the group's entries on levels before t +
//     (r - first rank of the group), since every earlier rank of the group
//     has at least as many tiles.
__global__ __launch_bounds__(1024) void varlen_schedule_grouped_kernel(const int* cu, int nseq, int tile,
                                                                      int levels, int ascending, int group,
                                                                      int* list, int n_entries) {
  __shared__ unsigned long long key[kListSortMax];
  __shared__ int gsum[kListSortMax];
  __shared__ int part[1024];
  const int tid = threadIdx.x;
  int P = 1;
  while (P < nseq) P <<= 1;
  for (int i = tid; i < P; i += 1024) {
    unsigned long long kv = ~0ULL;
    if (i < nseq) {
      const int len = cu[i + 1] - cu[i];
      const unsigned nt = len > 0 ? (unsigned)min((len + tile - 1) / tile, levels) : 0u;
      kv = ((unsigned long long)(0x7fffffffu - nt) << 32) | (unsigned)i;
    }
    key[i] = kv;
  }
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < P; i += 1024) {
        const int l = i ^ j;
        if (l > i) {
          const unsigned long long a = key[i], b = key[l];
          const bool up = (i & k) == 0;
          if ((a > b) == up) {
            key[i] = b;
            key[l] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  auto nt_of = [&](int r) { return (int)(0x7fffffffu - (unsigned)(key[r] >> 32)); };
  const int ng = (nseq + group - 1) / group;
  for (int g = tid; g < ng; g += 1024) {
    int n = 0;
    for (int r = g * group; r < min(nseq, (g + 1) * group); ++r) n += nt_of(r);
    gsum[g] = n;
  }
  __syncthreads();
  // exclusive prefix over the groups: each thread scans a contiguous run
  const int per = (ng + 1023) / 1024;
  const int g0 = min(ng, tid * per), g1 = min(ng, g0 + per);
  int run = 0;
  for (int g = g0; g < g1; ++g) run += gsum[g];
  part[tid] = run;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int acc = part[tid] - run;
  for (int g = g0; g < g1; ++g) {
    const int n = gsum[g];
    gsum[g] = acc;
    acc += n;
  }
  const int total = part[1023];
  __syncthreads();
  for (int r = tid; r < nseq; r += 1024) {
    const int nt = nt_of(r);
    if (nt == 0) continue;
    const int g = r / group, r0 = g * group, r1 = min(nseq, r0 + group);
    const int sq = (int)(key[r] & 0xffffffffu);
    for (int t = 0; t < nt; ++t) {
      int pos = gsum[g] + (r - r0);
      for (int m = r0; m < r1; ++m) {
        const int nm = nt_of(m);
        pos += ascending ? min(t, nm) : max(0, nm - 1 - t);
      }
      if (pos < n_entries) {  // cu_seqlens inconsistent with the totals: no write past the list
        list[2 * pos] = sq;
        list[2 * pos + 1] = t;
      }
    }
  }
  for (int e = total + tid; e < n_entries; e += 1024) {
    list[2 * e] = -1;
    list[2 * e + 1] = -1;
  }
}

int varlen_schedule(const int* cu, int nseq, int tile, int levels, bool ascending, int heads, int* list,
                    long long n_entries, hipStream_t st) {
  if (n_entries > 0x3fffffffLL || levels < 0) return FA_ERR_UNSUPPORTED;
  if (nseq <= kListSortMax) {
    hipLaunchKernelGGL(varlen_schedule_grouped_kernel, dim3(1), dim3(1024), 0, st, cu, nseq, tile, levels,
                       ascending ? 1 : 0, varlen_list_group(heads), list, (int)n_entries);
  } else {
    hipLaunchKernelGGL(varlen_schedule_kernel, dim3(1), dim3(1024), 0, st, cu, nseq, tile, levels,
                       ascending ? 1 : 0, list, (int)n_entries);
  }
  return launch_status();
}

// Row strides (elements between consecutive tokens) of q, of k and v, and
// of out; 0 = the contiguous layout (Hq * D, Hkv * D, Hq * D).
struct RowStrides {
  int q, kv, o;
};

static int fwd_dense(const void* q, const void* k, const void* v, void* out, float* lse,
                     int B, int Sq, int Sk, int Hq, int Hkv, int D, int dtype,
                     float scale, int causal, int window_left, int window_right, float softcap,
                     const float* alibi_slopes, const DropSpec& drop, void* stream,
                     RowStrides rs = RowStrides{0, 0, 0}) {
  int st = check_common(Hq, Hkv, D, dtype, scale, window_left, window_right, softcap);
  if (st) return st;
  if (B < 1 || Sq < 1 || Sk < 1) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return FA_ERR_INVALID_ARG;
  if (lse && !aligned4(lse)) return FA_ERR_INVALID_ARG;
  if (alibi_slopes && !aligned4(alibi_slopes)) return FA_ERR_INVALID_ARG;
  FwdParams prm{};
  prm.q = (const uint16_t*)q;
  prm.k = (const uint16_t*)k;
  prm.v = (const uint16_t*)v;
  prm.o = (uint16_t*)out;
  prm.lse = lse;
  prm.Sq = Sq;
  prm.Sk = Sk;
  prm.Hq = Hq;
  prm.g = Hq / Hkv;
  prm.q_rstride = rs.q ? rs.q : Hq * D;
  prm.k_rstride = rs.kv ? rs.kv : Hkv * D;
  prm.o_rstride = rs.o ? rs.o : Hq * D;
  prm.alibi = alibi_slopes;
  prm.wl = window_left;
  prm.wr = window_right;
  prm.drop = drop;
  return run_fwd(prm, D, dtype, scale, softcap, causal, Sq, B, (hipStream_t)stream);
}

static int fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                      const int* cu_seqlens_q, const int* cu_seqlens_k, int nseq,
                      int max_seqlen_q, int max_seqlen_k, int total_q, int total_k,
                      int Hq, int Hkv, int D, int dtype,
                      float scale, int causal, int window_left, int window_right, float softcap,
                      const float* alibi_slopes, const DropSpec& drop, void* workspace,
                      size_t workspace_bytes, void* stream) {
  int st = check_common(Hq, Hkv, D, dtype, scale, window_left, window_right, softcap);
  if (st) return st;
  if (nseq < 1 || max_seqlen_q < 0 || max_seqlen_k < 0 || total_q < 0 || total_k < 0) return FA_ERR_INVALID_ARG;
  if (!aligned4(cu_seqlens_q) || !aligned4(cu_seqlens_k)) return FA_ERR_INVALID_ARG;
  // tensors of an empty side (no queries at all, or no keys at all) may be NULL
  if (total_q > 0 && (!aligned16(q) || !aligned16(out))) return FA_ERR_INVALID_ARG;
  if (total_k > 0 && (!aligned16(k) || !aligned16(v))) return FA_ERR_INVALID_ARG;
  if (lse && !aligned4(lse)) return FA_ERR_INVALID_ARG;
  if (alibi_slopes && !aligned4(alibi_slopes)) return FA_ERR_INVALID_ARG;
  const size_t need = fa_fwd_varlen_workspace_size(nseq, total_q, Hq, D);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace))) return FA_ERR_WORKSPACE;
  if (max_seqlen_q == 0 || total_q == 0) return FA_OK;
  // the real (sequence, 128-row tile) pairs, heaviest level first
  const long long entries = varlen_list_entries(total_q, nseq, 128);
  st = varlen_schedule(cu_seqlens_q, nseq, 128, (max_seqlen_q + 127) / 128, false, Hq, (int*)workspace, entries,
                       (hipStream_t)stream);
  if (st) return st;
  FwdParams prm{};
  prm.tiles = (const int*)workspace;
  prm.q = (const uint16_t*)q;
  prm.k = (const uint16_t*)k;
  prm.v = (const uint16_t*)v;
  prm.o = (uint16_t*)out;
  prm.lse = lse;
  prm.cu_q = cu_seqlens_q;
  prm.cu_k = cu_seqlens_k;
  prm.Hq = Hq;
  prm.g = Hq / Hkv;
  prm.total_q = total_q;
  prm.q_rstride = Hq * D;
  prm.k_rstride = Hkv * D;
  prm.o_rstride = Hq * D;
  prm.alibi = alibi_slopes;
  prm.wl = window_left;
  prm.wr = window_right;
  prm.drop = drop;
  return run_fwd(prm, D, dtype, scale, softcap, causal, max_seqlen_q, nseq, (hipStream_t)stream, false, entries);
}

}  // namespace fa

using namespace fa;

extern "C" int fa_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                      int B, int Sq, int Sk, int Hq, int Hkv, int D, int dtype,
                      float scale, int causal, int window_left, int window_right, float softcap,
                      const float* alibi_slopes, void* stream) {
  return fwd_dense(q, k, v, out, lse, B, Sq, Sk, Hq, Hkv, D, dtype, scale, causal, window_left,
                   window_right, softcap, alibi_slopes, DropSpec{}, stream);
}

extern "C" int fa_fwd_dropout(const void* q, const void* k, const void* v, void* out, float* lse,
                              int B, int Sq, int Sk, int Hq, int Hkv, int D, int dtype,
                              float scale, int causal, int window_left, int window_right, float softcap,
                              const float* alibi_slopes, float dropout_p, unsigned long long seed,
                              unsigned long long offset, void* stream) {
  DropSpec drop;
  if (!make_drop(dropout_p, seed, offset, drop)) return FA_ERR_INVALID_ARG;
  return fwd_dense(q, k, v, out, lse, B, Sq, Sk, Hq, Hkv, D, dtype, scale, causal, window_left,
                   window_right, softcap, alibi_slopes, drop, stream);
}

extern "C" int fa_fwd_qkvpacked(const void* qkv, void* out, float* lse, int B, int S, int H, int D,
                                int dtype, float scale, int causal, int window_left, int window_right,
                                float softcap, const float* alibi_slopes, void* stream) {
  if (!aligned16(qkv) || H < 1 || D < 1) return FA_ERR_INVALID_ARG;
  const uint16_t* base = (const uint16_t*)qkv;
  const int hd = H * D;
  return fwd_dense(base, base + hd, base + 2 * hd, out, lse, B, S, S, H, H, D, dtype, scale, causal,
                   window_left, window_right, softcap, alibi_slopes, DropSpec{}, stream,
                   RowStrides{3 * hd, 3 * hd, hd});
}

extern "C" int fa_fwd_kvpacked(const void* q, const void* kv, void* out, float* lse,
                               int B, int Sq, int Sk, int Hq, int Hkv, int D, int dtype,
                               float scale, int causal, int window_left, int window_right, float softcap,
                               const float* alibi_slopes, void* stream) {
  if (!aligned16(kv) || Hkv < 1 || D < 1) return FA_ERR_INVALID_ARG;
  const uint16_t* base = (const uint16_t*)kv;
  return fwd_dense(q, base, base + Hkv * D, out, lse, B, Sq, Sk, Hq, Hkv, D, dtype, scale, causal,
                   window_left, window_right, softcap, alibi_slopes, DropSpec{}, stream,
                   RowStrides{0, 2 * Hkv * D, 0});
}

extern "C" size_t fa_fwd_fp8_workspace_size(int B, int Sk, int Hkv, int D) {
  if (B < 1 || Sk < 1 || Hkv < 1 || D < 1) return 0;
  return align_up((size_t)B * Sk * Hkv * D * 2, 256);
}

extern "C" int fa_fwd_fp8(const void* q, const void* k, const void* v, void* out, float* lse,
                          int B, int Sq, int Sk, int Hq, int Hkv, int D,
                          float scale, int causal, int window_left, int window_right, float softcap,
                          const float* alibi_slopes, const float* descale_q, const float* descale_k,
                          const float* descale_v, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_common(Hq, Hkv, D, FA_DTYPE_BF16, scale, window_left, window_right, softcap);
  if (st) return st;
  if (B < 1 || Sq < 1 || Sk < 1) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return FA_ERR_INVALID_ARG;
  if (lse && !aligned4(lse)) return FA_ERR_INVALID_ARG;
  if (alibi_slopes && !aligned4(alibi_slopes)) return FA_ERR_INVALID_ARG;
  if ((descale_q && !aligned4(descale_q)) || (descale_k && !aligned4(descale_k)) ||
      (descale_v && !aligned4(descale_v)))
    return FA_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
  const size_t need = fa_fwd_fp8_workspace_size(B, Sk, Hkv, D);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return FA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  // V: fp8 -> bfloat16 copy in the workspace (exact)
  const int64_t n16 = (int64_t)B * Sk * Hkv * D / 16;
  hipLaunchKernelGGL(fp8_to_bf16_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, s,
                     (const uint8_t*)v, (uint16_t*)workspace, n16);
  FwdParams prm{};
  prm.q = (const uint16_t*)q;  // fp8 bytes, read as such by the FP8 kernel
  prm.k = (const uint16_t*)k;
  prm.v = (const uint16_t*)workspace;
  prm.o = (uint16_t*)out;
  prm.lse = lse;
  prm.Sq = Sq;
  prm.Sk = Sk;
  prm.Hq = Hq;
  prm.g = Hq / Hkv;
  prm.q_rstride = Hq * D;
  prm.k_rstride = Hkv * D;
  prm.o_rstride = Hq * D;
  prm.alibi = alibi_slopes;
  prm.wl = window_left;
  prm.wr = window_right;
  prm.dsc_q = descale_q;
  prm.dsc_k = descale_k;
  prm.dsc_v = descale_v;
  return run_fwd(prm, D, FA_DTYPE_BF16, scale, softcap, causal, Sq, B, s, true);
}

extern "C" size_t fa_fwd_varlen_workspace_size(int nseq, int total_q, int Hq, int D) {
  (void)Hq;
  (void)D;
  if (nseq < 1 || total_q < 1) return 0;
  return varlen_list_bytes(total_q, nseq, 128);
}

extern "C" int fa_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                             const int* cu_seqlens_q, const int* cu_seqlens_k, int nseq,
                             int max_seqlen_q, int max_seqlen_k, int total_q, int total_k,
                             int Hq, int Hkv, int D, int dtype,
                             float scale, int causal, int window_left, int window_right, float softcap,
                             const float* alibi_slopes, void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_varlen(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, nseq, max_seqlen_q, max_seqlen_k,
                    total_q, total_k, Hq, Hkv, D, dtype, scale, causal, window_left, window_right, softcap,
                    alibi_slopes, DropSpec{}, workspace, workspace_bytes, stream);
}

extern "C" int fa_fwd_varlen_dropout(const void* q, const void* k, const void* v, void* out, float* lse,
                                     const int* cu_seqlens_q, const int* cu_seqlens_k, int nseq,
                                     int max_seqlen_q, int max_seqlen_k, int total_q, int total_k,
                                     int Hq, int Hkv, int D, int dtype,
                                     float scale, int causal, int window_left, int window_right,
                                     float softcap, const float* alibi_slopes, float dropout_p,
                                     unsigned long long seed, unsigned long long offset, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  DropSpec drop;
  if (!make_drop(dropout_p, seed, offset, drop)) return FA_ERR_INVALID_ARG;
  return fwd_varlen(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, nseq, max_seqlen_q, max_seqlen_k,
                    total_q, total_k, Hq, Hkv, D, dtype, scale, causal, window_left, window_right, softcap,
                    alibi_slopes, drop, workspace, workspace_bytes, stream);
}
