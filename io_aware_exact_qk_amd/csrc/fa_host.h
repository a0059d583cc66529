// fa_host.h — host-side helpers shared by the entry points: argument checks,
// launch-grid remapping for the 8 XCDs, and the kernel-timing hooks.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "fa.h"

namespace fa {

inline bool aligned16(const void* p) { return p && (((uintptr_t)p) & 15u) == 0; }
inline bool opt_aligned16(const void* p) { return p == nullptr || aligned16(p); }
inline bool aligned4(const void* p) { return p && (((uintptr_t)p) & 3u) == 0; }

// Checks shared by the dense and packed entry points.
inline int check_common(int Hq, int Hkv, int D, int dtype, float scale, int wl, int wr,
                        float softcap) {
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16) return FA_ERR_INVALID_ARG;
  if (D < 1) return FA_ERR_INVALID_ARG;
  if (!(scale > 0.0f) || !isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (wl < -1 || wr < -1) return FA_ERR_INVALID_ARG;
  if (!(softcap >= 0.0f) || !isfinite(softcap)) return FA_ERR_INVALID_ARG;
  if (D != 32 && D != 64 && D != 96 && D != 128 && D != 256) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Dropout parameters of one call (see the dropout section of fa_device.h).
struct DropSpec {
  uint32_t k0, k1;  // seed, low and high word
  uint32_t off;     // counter word 3
  uint32_t t;       // byte threshold, round(256 p); 0 = no dropout
  float scale;      // 256 / (256 - t)
};

// Dropout parameters: p in [0, 255.5/256), finite.  The byte threshold is
// t = round(256 p) with ties to even (the default rounding mode of lrint);
// t = 0 means no dropout.  The seed is the generator key, the low word of
// the offset its counter word 3.
inline bool make_drop(float p, unsigned long long seed, unsigned long long offset, DropSpec& d) {
  if (!(p >= 0.0f) || !(p < 255.5f / 256.0f)) return false;
  const long t = lrintf(p * 256.0f);
  d.k0 = (uint32_t)(seed & 0xffffffffull);
  d.k1 = (uint32_t)(seed >> 32);
  d.off = (uint32_t)(offset & 0xffffffffull);
  d.t = (uint32_t)t;
  d.scale = 256.0f / (float)(256 - t);
  return true;
}

// Work-group ids are handed to the 8 XCDs round-robin (id % 8).
struct TileId {
  int t, h, b;  // tile index along the sequence, head, batch entry
};

// Logical coordinates of this work-group.
//  * default: the hardware id is remapped so that each XCD receives one
//    contiguous block of logical tiles, which keeps tiles that share K/V (or
//    Q/dO) rows on the same L2;
//  * balanced (causal launches, where tiles differ a lot in work): tiles are
//    taken level by level (tile index), so the heaviest tile of every
//    (head, batch) pair is dispatched first.  Work-groups go to the 8 XCDs
//    round-robin (hardware id mod 8), so XCD x serves the pairs
//    p = x (mod 8), and with `group` > 0 it serves them `group` pairs at a
//    time: all levels of one group of pairs, heaviest first, before the
//    next group.  Tiles that share a pair's K/V (or Q/dO) rows then run
//    together on one L2 instead of every pair of the XCD being in flight
//    at once.  heavy_last: the heaviest tile is the last one.
__device__ __forceinline__ TileId tile_id(int n_tiles, int n_heads, int n_batch, bool balanced,
                                          bool heavy_last, int group) {
  TileId r;
  const int hw = (int)blockIdx.x;
  int t;
  if (balanced) {
    const int np = n_heads * n_batch;
    int pair;
    if (group > 0 && (np & 7) == 0) {
      const int x = hw & 7, j = hw >> 3;  // XCD, dispatch order on it
      const int per = np >> 3;            // pairs of this XCD
      const int gsz = group * n_tiles;    // tiles of a full group
      const int gi = j / gsz;
      const int g0 = gi * group;
      const int gn = min(group, per - g0);  // pairs of this group
      const int rr = j - gi * gsz;
      t = rr / gn;
      pair = x + 8 * (g0 + rr % gn);
    } else {
      pair = hw % np;
      t = hw / np;
    }
    r.h = pair % n_heads;
    r.b = pair / n_heads;
  } else {
    const int n = n_tiles * n_heads * n_batch;
    const int per = n / 8;
    const int id = (hw >= per * 8) ? hw : (hw & 7) * per + (hw >> 3);
    t = id % n_tiles;
    r.h = (id / n_tiles) % n_heads;
    r.b = id / (n_tiles * n_heads);
  }
  r.t = heavy_last ? n_tiles - 1 - t : t;
  return r;
}

// Pairs per XCD group of a balanced launch.  Measured on the causal
// fwd+bwd sweep (bf16, H = 16, D = 128, B*S = 16384) against no grouping:
// 8 pairs per group takes 10% off the time at S = 512 (64 pairs per XCD),
// 17% at 1K, 4% at 2K, and leaves S >= 4K (8 pairs or fewer per XCD)
// unchanged; 1 or 2 pairs per group are slower at S >= 2K, where the last
// group's heaviest tiles then start too late to finish with the rest.
constexpr int kTileGroup = 8;

// ---- varlen tile list (kernels in fa_fwd.hip) ----
// A packed variable-length launch runs one work-group per (list entry, head)
// instead of one per (max_seqlen tile, head, sequence): the list holds the
// real (sequence, tile) pairs only, built on the device from cu_seqlens.
// Entry e is the int pair list[2e] = sequence, list[2e + 1] = tile index
// within it; unused trailing entries hold -1.  Order, for nseq <=
// kListSortMax: the sequences sorted by tile count, most first (ties: lower
// index first), cut into groups of varlen_list_group(heads) sequences; each
// group level by level (tile index t from the highest down, or from 0 up
// with ascending), sequences in sorted order within a level.  Heavy tiles
// of a causal launch (the last query tiles, or the first key tiles) of the
// longest sequences come first, and each XCD (work-group id mod 8, so heads
// h = x mod 8 when heads is a multiple of 8) holds about four (sequence,
// head) pairs in flight.  Measured at 16 heads (causal fwd+bwd) against
// groups of 1, 3, 4, 8, 16 and all sequences: 2 sequences per group is best
// or within noise of the best on 13 sequences of 448-4002 tokens, 16 of 2048
// and 64 of 128-1024.  More sequences: level by level over all sequences,
// index order within a level.
constexpr int kListSortMax = 4096;
inline int varlen_list_group(int heads) { return heads >= 32 ? 1 : 32 / (heads > 0 ? heads : 1); }

// Entries a list of `tile`-row tiles needs at most: sum_s ceil(L_s / tile)
// <= (total + nseq (tile - 1)) / tile.
inline long long varlen_list_entries(long long total, int nseq, int tile) {
  return (total + (long long)nseq * (tile - 1)) / tile;
}

inline size_t varlen_list_bytes(long long total, int nseq, int tile) {
  return align_up((size_t)varlen_list_entries(total, nseq, tile) * 2 * sizeof(int), 256);
}

// Enqueues the list build: cu (nseq + 1) prefix sums of the lengths on the
// device, levels = ceil(max_len / tile) (tiles past it are not listed).
int varlen_schedule(const int* cu, int nseq, int tile, int levels, bool ascending, int heads, int* list,
                    long long n_entries, hipStream_t st);

// Work-group of a list launch: entry blockIdx.x / n_heads, head
// blockIdx.x % n_heads.  Returns false for an unused entry (uniform over the
// work-group).
__device__ __forceinline__ bool tile_from_list(const int* list, int n_heads, TileId& r) {
  const int e = (int)blockIdx.x / n_heads;
  r.h = (int)blockIdx.x % n_heads;
  r.b = list[2 * e];
  r.t = list[2 * e + 1];
  return r.b >= 0;
}

// ---- kernel timing (implemented in fa_api.hip) ----
void prof_before(int kind, hipStream_t s);
void prof_after(int kind, hipStream_t s);

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace fa
