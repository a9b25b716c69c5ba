// C ABI of libattn.so (declared in include/attn.h): argument validation,
// kernel selection and launch geometry.  Everything here runs on the host;
// every check happens before the first HIP call, so an invalid call enqueues
// nothing and touches no memory.
#include "attn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <initializer_list>
#include <cmath>
#include <cstdint>
#include <cstdlib>

#include "launch.hpp"

namespace {

constexpr int kPrefillRows = 256;  // query rows per prefill workgroup
constexpr int64_t kSmallGridBlocks = 128;  // 256-row grids this small use 128-row blocks (half the 256 CUs)
// packed batches whose mean query length is at most this many rows use
// 128-row blocks, two workgroups per CU: their blocks are short, and a CU
// running two overlaps one block's Q/K/V loads and O stores with the other's
// loop (measured faster up to a mean of ~4k rows, even at ~8k)
constexpr int64_t kPackedShortMeanRows = 6144;
constexpr int kDecodeTile = 128;   // cache rows per decode tile
constexpr int kDecodeMaxHeads = 16;
constexpr int kDecodeMaxSplits = 64;     // partials one combine merges
constexpr int kDecodeTargetWorkgroups = 512;  // decode workgroups that fill MI355X (2 per CU)
// with per-sequence lengths, default chunks hold at most this many tiles (768
// rows): the chunks covering a sequence then number in proportion to its
// length and the last workgroups to finish hold little work
constexpr int kDecodeVarlenChunkTiles = 6;
constexpr int kDecodePartPad = 4;       // floats ahead of o[D] in a per-head partial
constexpr float kLog2e = 1.4426950408889634f;

// Polls a wait of the prefill's counted KV ring (masked grids) makes before
// it gives up and the workgroup writes its rows as NaN.  A correct run never
// comes near the default; the environment variable ATTN_RING_POLL_LIMIT
// (read on every call, clamped to [1, 2^18]) lowers it, so that tests can
// drive that path.
inline int ring_poll_limit() {
  constexpr int kDefault = 1 << 18;
  const char* e = std::getenv("ATTN_RING_POLL_LIMIT");
  if (e == nullptr || *e == 0) return kDefault;
  const long v = std::strtol(e, nullptr, 10);
  return (int)std::min<long>(std::max<long>(v, 1), kDefault);
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// head-dim stride 1; other strides non-negative multiples of 8 elements (16 bytes)
inline bool strides_ok(const attn_strides& s) {
  return s.d == 1 && s.b >= 0 && s.h >= 0 && s.n >= 0 && s.b % 8 == 0 && s.h % 8 == 0 && s.n % 8 == 0;
}

// An output view whose elements are all distinct addresses: taken in order
// of stride, every dimension of extent > 1 steps at least past the span of
// the dimensions below it.  Views that alias rows or heads would have several
// workgroups store to one address, so they are refused rather than raced.
struct Dim {
  int64_t extent, stride;
};
inline bool writes_once(std::initializer_list<Dim> dims) {
  Dim d[4];
  int n = 0;
  for (const Dim& x : dims)
    if (x.extent > 1) d[n++] = x;
  std::sort(d, d + n, [](const Dim& a, const Dim& b) { return a.stride < b.stride; });
  int64_t span = 1;  // max offset + 1 over the dimensions taken so far
  for (int i = 0; i < n; ++i) {
    if (d[i].stride < span) return false;
    span += (d[i].extent - 1) * d[i].stride;
  }
  return true;
}

inline bool dtype_ok(attn_dtype t) { return t == ATTN_F16 || t == ATTN_BF16; }

inline uint32_t q_sign_mask(float scale) { return std::signbit(scale) ? 0x80008000u : 0u; }

// Scores are scaled by c = |scale| log2(e) after the sign is folded into Q.  A
// zero scale becomes a tiny positive c: every visible score is then ~0 (to far
// below fp32 resolution) while masked keys still map to -inf, not to NaN.
inline float score_coef(float scale) {
  const float c = std::fabs(scale) * kLog2e;
  return c > 0.f ? c : 1e-30f;
}

// Per-lane buffer offsets inside a tile must fit in 31 bits.
constexpr int64_t kMaxRowStride = int64_t(1) << 22;

inline int64_t slice_bytes(int64_t rows, int64_t stride_n, int D) { return ((rows - 1) * stride_n + D) * 2; }

struct DecodeGeometry {
  int hgroups, heads_per_wg, max_splits;
  size_t part_bytes;
};

DecodeGeometry decode_geometry(int B, int Hq, int Hkv, int S_max, int D) {
  DecodeGeometry g{};
  const int group = Hq / Hkv;
  g.hgroups = (group + kDecodeMaxHeads - 1) / kDecodeMaxHeads;
  g.heads_per_wg = (group + g.hgroups - 1) / g.hgroups;
  const int tiles = (S_max + kDecodeTile - 1) / kDecodeTile;
  g.max_splits = tiles < kDecodeMaxSplits ? tiles : kDecodeMaxSplits;
  const size_t slots = (size_t)B * Hkv * g.hgroups;
  g.part_bytes = slots * (size_t)g.max_splits * g.heads_per_wg * (size_t)(D + kDecodePartPad) * sizeof(float);
  return g;
}

}  // namespace

extern "C" {

const char* attn_status_string(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "invalid shape (size <= 0, Hq % Hkv != 0, or position/length out of range)";
    case ATTN_ERR_UNSUPPORTED: return "unsupported argument (head dim, dtype, stride, alignment or scale)";
    case ATTN_ERR_WORKSPACE: return "decode workspace missing or too small";
    case ATTN_ERR_HIP: return "HIP runtime error at launch";
  }
  return "unknown status";
}

// the kernels' mask: mode 0 none, 1 causal, 2 band; the diagonal aligned
// top-left (query i at key position i) or bottom-right (i + Nkv - Nq)
struct MaskSpec {
  int mode, bottom_right, left, right;
};

// attn_fwd's causal argument as a mask (mode -1: not a valid value)
static MaskSpec mask_of_causal(int causal) {
  if (causal < ATTN_CAUSAL_NONE || causal > ATTN_CAUSAL_BOTTOM_RIGHT) return MaskSpec{-1, 0, -1, -1};
  return MaskSpec{causal != ATTN_CAUSAL_NONE ? 1 : 0, causal == ATTN_CAUSAL_BOTTOM_RIGHT ? 1 : 0, -1,
                  causal != ATTN_CAUSAL_NONE ? 0 : -1};
}

// an attn_mask as the kernels' mask (mode -1: not a valid value)
static MaskSpec mask_of(attn_mask m) {
  if ((m.align != ATTN_ALIGN_TOP_LEFT && m.align != ATTN_ALIGN_BOTTOM_RIGHT) || m.window_left < -1 ||
      m.window_right < -1)
    return MaskSpec{-1, 0, -1, -1};
  const int mode = (m.window_left < 0 && m.window_right < 0) ? 0 : (m.window_left < 0 && m.window_right == 0) ? 1 : 2;
  return MaskSpec{mode, m.align == ATTN_ALIGN_BOTTOM_RIGHT ? 1 : 0, m.window_left, m.window_right};
}

// Band sides that hide nothing become open (-1), so the mask takes its
// cheapest mode.  A query's key position p = i + off lies in [Nkv - Nq, Nkv)
// bottom-right and [0, Nq) top-left, keys in [0, Nkv): with a side of at least
// reach = max(Nq, Nkv) every key passes that side's test for every query.
// (Packed batches pass the totals, which bound every sequence's lengths.)
static MaskSpec open_wide_sides(MaskSpec mk, int64_t reach) {
  if (mk.mode != 2) return mk;
  if (mk.left >= reach) mk.left = -1;
  if (mk.right >= reach) mk.right = -1;
  mk.mode = (mk.left < 0 && mk.right < 0) ? 0 : (mk.left < 0 && mk.right == 0) ? 1 : 2;
  return mk;
}

// The kernels evaluate band bounds as 32-bit sums of a position, a window
// side (open sides count as 2^30) and a tile offset; sequences up to 2^28 rows
// keep every such sum inside int32.
constexpr int64_t kMaxBandRows = int64_t(1) << 28;

static attn_status fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int Hq, int Hkv, int Nq, int Nkv, int D,
                            attn_strides sq, attn_strides sk, attn_strides sv, attn_strides so,
                            float scale, MaskSpec mk, attn_dtype dtype, void* stream) {
  if (!q || !k || !v || !o) return ATTN_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nkv <= 0 || D <= 0) return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if (!dtype_ok(dtype) || !std::isfinite(scale)) return ATTN_ERR_UNSUPPORTED;
  if (mk.mode < 0) return ATTN_ERR_UNSUPPORTED;
  mk = open_wide_sides(mk, Nq > Nkv ? Nq : Nkv);
  if (mk.mode == 2 && (Nq > kMaxBandRows || Nkv > kMaxBandRows)) return ATTN_ERR_UNSUPPORTED;
  if (!strides_ok(sq) || !strides_ok(sk) || !strides_ok(sv) || !strides_ok(so)) return ATTN_ERR_UNSUPPORTED;
  if (!writes_once({{B, so.b}, {Hq, so.h}, {Nq, so.n}, {D, 1}})) return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_ERR_UNSUPPORTED;
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return ATTN_ERR_UNSUPPORTED;
  if (sq.n > kMaxRowStride || sk.n > kMaxRowStride || sv.n > kMaxRowStride) return ATTN_ERR_UNSUPPORTED;
  // 256 query rows per workgroup (8 waves, two per SIMD), or 128 (4 waves,
  // one per SIMD) when 256-row blocks would leave at least half the CUs idle
  const int64_t nqb256 = ((int64_t)Nq + kPrefillRows - 1) / kPrefillRows;
  const int rows = nqb256 * Hq * B <= kSmallGridBlocks ? kPrefillRows / 2 : kPrefillRows;
  const int64_t nqb = ((int64_t)Nq + rows - 1) / rows;
  const int64_t nblocks = nqb * Hq * B;
  if (nblocks > INT_MAX) return ATTN_ERR_SHAPE;

  attn::FwdArgs a{};
  a.ring_polls = ring_poll_limit();
  a.rows = rows;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.sqb = sq.b; a.sqh = sq.h; a.sqn = sq.n;
  a.skb = sk.b; a.skh = sk.h; a.skn = sk.n;
  a.svb = sv.b; a.svh = sv.h; a.svn = sv.n;
  a.sob = so.b; a.soh = so.h; a.son = so.n;
  a.Hq = Hq; a.Hkv = Hkv; a.Nq = Nq; a.Nkv = Nkv; a.group = Hq / Hkv;
  a.nqb = (int)nqb;
  a.nblocks = (int)nblocks;
  // XCD-aware remap: blocks are dispatched round-robin over 8 XCDs; remapping
  // gives each XCD a contiguous run of (kv head, query block) work.  Only used
  // when every XCD then gets whole kv-head units, or (non-causal, equal-length
  // blocks) an equal slice of one unit.
  const int64_t per_xcd = nblocks / 8;
  const int64_t per_unit = (int64_t)a.group * nqb;
  a.remap = (nblocks % 8 == 0) && per_xcd > 0 &&
            ((per_xcd % per_unit == 0) || (mk.mode == 0 && per_unit % per_xcd == 0));
  a.causal_off = mk.bottom_right ? Nkv - Nq : 0;
  a.win_left = mk.left;
  a.win_right = mk.right;
  a.c = score_coef(scale);
  a.qsign = q_sign_mask(scale);
  a.q_bytes = slice_bytes(Nq, sq.n, D);
  a.k_bytes = slice_bytes(Nkv, sk.n, D);
  a.v_bytes = slice_bytes(Nkv, sv.n, D);

  a.units = B * Hkv;

  const hipError_t e =
      attn::launch_prefill(a, D, dtype == ATTN_BF16, mk.mode, false, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int Hq, int Hkv, int Nq, int Nkv, int D,
                     attn_strides sq, attn_strides sk, attn_strides sv, attn_strides so,
                     float scale, int causal, attn_dtype dtype, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, sq, sk, sv, so, scale, mask_of_causal(causal), dtype,
                  stream);
}

attn_status attn_fwd_masked(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int Hq, int Hkv, int Nq, int Nkv, int D,
                            attn_strides sq, attn_strides sk, attn_strides sv, attn_strides so,
                            float scale, attn_mask mask, attn_dtype dtype, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, sq, sk, sv, so, scale, mask_of(mask), dtype, stream);
}

static attn_status fwd_varlen_impl(const void* q, const void* k, const void* v, void* o, float* lse,
                                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B,
                                   int max_seqlen_q, int total_q, int total_k, int Hq, int Hkv, int D,
                                   attn_strides sq, attn_strides sk, attn_strides sv, attn_strides so,
                                   float scale, MaskSpec mk, attn_dtype dtype, void* stream) {
  if (!q || !k || !v || !o || !cu_seqlens_q || !cu_seqlens_k) return ATTN_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || max_seqlen_q <= 0 || total_q <= 0 || total_k < 0 || D <= 0)
    return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if (!dtype_ok(dtype) || !std::isfinite(scale)) return ATTN_ERR_UNSUPPORTED;
  if (mk.mode < 0) return ATTN_ERR_UNSUPPORTED;
  mk = open_wide_sides(mk, total_q > total_k ? total_q : total_k);
  if (mk.mode == 2 && (total_q > kMaxBandRows || total_k > kMaxBandRows)) return ATTN_ERR_UNSUPPORTED;
  // packed (token, head, dim) views: the batch stride is unused and not checked
  attn_strides sq3 = sq, sk3 = sk, sv3 = sv, so3 = so;
  sq3.b = sk3.b = sv3.b = so3.b = 0;
  if (!strides_ok(sq3) || !strides_ok(sk3) || !strides_ok(sv3) || !strides_ok(so3)) return ATTN_ERR_UNSUPPORTED;
  if (!writes_once({{total_q, so.n}, {Hq, so.h}, {D, 1}})) return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_ERR_UNSUPPORTED;
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return ATTN_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3u) || (reinterpret_cast<uintptr_t>(cu_seqlens_k) & 3u))
    return ATTN_ERR_UNSUPPORTED;
  if (sq.n > kMaxRowStride || sk.n > kMaxRowStride || sv.n > kMaxRowStride) return ATTN_ERR_UNSUPPORTED;
  const int rows = (int64_t)total_q <= kPackedShortMeanRows * B ? kPrefillRows / 2 : kPrefillRows;
  const int64_t nqb = ((int64_t)max_seqlen_q + rows - 1) / rows;
  const int64_t units = (int64_t)B * Hkv;
  const int64_t group = Hq / Hkv;
  // units rounded up to a multiple of the 8 XCDs (the extra workgroups exit)
  const int64_t nblocks = (units + 7) / 8 * 8 * group * nqb;
  if (nblocks > INT_MAX) return ATTN_ERR_SHAPE;

  attn::FwdArgs a{};
  a.ring_polls = ring_poll_limit();
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.sqh = sq.h; a.sqn = sq.n;
  a.skh = sk.h; a.skn = sk.n;
  a.svh = sv.h; a.svn = sv.n;
  a.soh = so.h; a.son = so.n;
  a.Hq = Hq; a.Hkv = Hkv; a.group = (int)group;
  a.Nq = max_seqlen_q;  // per-sequence query rows are capped at this bound
  a.rows = rows;
  a.nqb = (int)nqb;
  a.nblocks = (int)nblocks;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.total_q = total_q;
  a.total_k = total_k;
  a.units = (int)units;
  a.causal_br = mk.bottom_right;
  a.win_left = mk.left;
  a.win_right = mk.right;
  a.c = score_coef(scale);
  a.qsign = q_sign_mask(scale);

  const hipError_t e =
      attn::launch_prefill(a, D, dtype == ATTN_BF16, mk.mode, true, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B, int max_seqlen_q,
                            int total_q, int total_k, int Hq, int Hkv, int D,
                            attn_strides sq, attn_strides sk, attn_strides sv, attn_strides so,
                            float scale, int causal, attn_dtype dtype, void* stream) {
  return fwd_varlen_impl(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, max_seqlen_q, total_q, total_k, Hq, Hkv,
                         D, sq, sk, sv, so, scale, mask_of_causal(causal), dtype, stream);
}

attn_status attn_fwd_varlen_masked(const void* q, const void* k, const void* v, void* o, float* lse,
                                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B,
                                   int max_seqlen_q, int total_q, int total_k, int Hq, int Hkv, int D,
                                   attn_strides sq, attn_strides sk, attn_strides sv, attn_strides so,
                                   float scale, attn_mask mask, attn_dtype dtype, void* stream) {
  return fwd_varlen_impl(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, max_seqlen_q, total_q, total_k, Hq, Hkv,
                         D, sq, sk, sv, so, scale, mask_of(mask), dtype, stream);
}

size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int S_max, int D) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || S_max <= 0 || D <= 0 || Hq % Hkv != 0) return 0;
  const DecodeGeometry g = decode_geometry(B, Hq, Hkv, S_max, D);
  return g.part_bytes;
}

namespace {

// a paged cache: page ids of sequence b at table[b * mbps ...], pages of
// 2^lg_ps rows, num_pages pages in the pools
struct PagedSpec {
  const int32_t* table;
  int mbps, lg_ps, num_pages;
};

// shared by attn_decode (lens == nullptr: every sequence has cache_len slots),
// attn_decode_varlen (sequence b has min(max(lens[b], 0), cache_len)) and
// attn_decode_paged (the same over a paged cache, pg != nullptr)
static attn_status decode_impl(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                        int B, int Hq, int Hkv, int S_max, int cache_len, const int32_t* lens, int D,
                        attn_strides sq, attn_strides skc, attn_strides svc, attn_strides so,
                        float scale, attn_dtype dtype, int num_splits,
                        void* workspace, size_t workspace_bytes, void* stream, const PagedSpec* pg = nullptr,
                        int window_left = -1, bool use_scratch = false) {
  if (!q || !k_cache || !v_cache || !o) return ATTN_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || S_max <= 0 || D <= 0) return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0 || cache_len < 1 || cache_len > S_max || num_splits < 0) return ATTN_ERR_SHAPE;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if (!dtype_ok(dtype) || !std::isfinite(scale)) return ATTN_ERR_UNSUPPORTED;
  // q and o are (B, H, D): their n stride is unused and not checked
  attn_strides sq3 = sq, so3 = so;
  sq3.n = 0;
  so3.n = 0;
  if (!strides_ok(sq3) || !strides_ok(skc) || !strides_ok(svc) || !strides_ok(so3)) return ATTN_ERR_UNSUPPORTED;
  if (!writes_once({{B, so.b}, {Hq, so.h}, {D, 1}})) return ATTN_ERR_UNSUPPORTED;
  if (skc.n > kMaxRowStride || svc.n > kMaxRowStride) return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o)) return ATTN_ERR_UNSUPPORTED;
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return ATTN_ERR_UNSUPPORTED;
  if (lens && (reinterpret_cast<uintptr_t>(lens) & 3u)) return ATTN_ERR_UNSUPPORTED;
  const DecodeGeometry g = decode_geometry(B, Hq, Hkv, S_max, D);
  if (!use_scratch && (!workspace || !aligned16(workspace) || workspace_bytes < g.part_bytes))
    return ATTN_ERR_WORKSPACE;
  // B * Hkv goes in grid x (limit 2^31 - 1) or z (limit 65535); head groups in y
  if ((int64_t)B * Hkv > 0x7fffffff || g.hgroups > 65535) return ATTN_ERR_SHAPE;

  if (window_left < -1) return ATTN_ERR_SHAPE;
  // tiles a chunk grid must cover: with a window a sequence's slots start at
  // the tile holding slot len - 1 - window_left, so at most window_left + 1
  // slots plus that tile's lead-in are read
  int tiles = (cache_len + kDecodeTile - 1) / kDecodeTile;
  if (window_left >= 0) {
    if (!lens) {
      const int kbeg = (cache_len - 1 - window_left > 0 ? cache_len - 1 - window_left : 0) & ~(kDecodeTile - 1);
      tiles = (cache_len - kbeg + kDecodeTile - 1) / kDecodeTile;
    } else {
      const int64_t span = ((int64_t)window_left + 2 * kDecodeTile - 1) / kDecodeTile;
      if (span < tiles) tiles = (int)span;
    }
  }
  // default: enough chunks for ~kDecodeTargetWorkgroups workgroups (two per CU,
  // each with two 128-row tiles in flight), at most max_splits per (batch, kv
  // head, head group)
  const int64_t slots = (int64_t)B * Hkv * g.hgroups;
  int want = num_splits > 0 ? num_splits : (int)((kDecodeTargetWorkgroups + slots - 1) / slots);
  if (num_splits == 0 && lens) {
    const int floor_splits = (tiles + kDecodeVarlenChunkTiles - 1) / kDecodeVarlenChunkTiles;
    if (want < floor_splits) want = floor_splits;
  }
  if (want > g.max_splits) want = g.max_splits;
  if (want > tiles) want = tiles;
  if (want < 1) want = 1;
  const int tiles_per_split = (tiles + want - 1) / want;
  const int nsplit = (tiles + tiles_per_split - 1) / tiles_per_split;

  attn::DecodeArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k_cache);
  a.v = static_cast<const uint16_t*>(v_cache);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.lens = lens;
  a.sqb = sq.b; a.sqh = sq.h;
  a.skb = skc.b; a.skh = skc.h; a.skn = skc.n;
  a.svb = svc.b; a.svh = svc.h; a.svn = svc.n;
  a.sob = so.b; a.soh = so.h;
  a.Hq = Hq; a.Hkv = Hkv; a.group = Hq / Hkv; a.cache_len = cache_len;
  a.heads_per_wg = g.heads_per_wg;
  a.hgroups = g.hgroups;
  a.nsplit = nsplit;
  a.max_splits = g.max_splits;
  a.rows_per_split = tiles_per_split * kDecodeTile;
  a.unit_fast = (lens != nullptr || (int64_t)B * Hkv > 65535) ? 1 : 0;
  a.c = score_coef(scale);
  a.qsign = q_sign_mask(scale);
  a.part = static_cast<float*>(workspace);
  if (use_scratch) {
    // the library's scratch holds exactly this call's partials: nsplit slots
    // per (batch, kv head, head group) rather than the workspace's max_splits
    a.max_splits = nsplit;
    const size_t need = nsplit > 1 ? (size_t)slots * nsplit * g.heads_per_wg * (size_t)(D + kDecodePartPad) *
                                         sizeof(float)
                                   : 0;
    if (need > ATTN_DECODE_NOALLOC_SCRATCH_BYTES) return ATTN_ERR_WORKSPACE;
    void* p = nullptr;
    if (attn::decode_scratch_address(static_cast<hipStream_t>(stream), &p) != hipSuccess) return ATTN_ERR_HIP;
    a.part = static_cast<float*>(p);
  }
  a.window_left = window_left;
  if (pg) {
    a.block_table = pg->table;
    a.mbps = pg->mbps;
    a.lg_ps = pg->lg_ps;
    a.num_pages = pg->num_pages;
  }

  const hipError_t e = attn::launch_decode(a, B, D, dtype == ATTN_BF16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // namespace

attn_status attn_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                        int B, int Hq, int Hkv, int S_max, int cache_len, int D,
                        attn_strides sq, attn_strides skc, attn_strides svc, attn_strides so,
                        float scale, attn_dtype dtype, int num_splits,
                        void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(q, k_cache, v_cache, o, lse, B, Hq, Hkv, S_max, cache_len, nullptr, D, sq, skc, svc, so,
                     scale, dtype, num_splits, workspace, workspace_bytes, stream);
}

attn_status attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                                int B, int Hq, int Hkv, int S_max, int cache_len, int D,
                                attn_strides sq, attn_strides skc, attn_strides svc, attn_strides so,
                                float scale, attn_dtype dtype, int num_splits, void* stream) {
  return decode_impl(q, k_cache, v_cache, o, lse, B, Hq, Hkv, S_max, cache_len, nullptr, D, sq, skc, svc, so,
                     scale, dtype, num_splits, nullptr, 0, stream, nullptr, -1, true);
}

attn_status attn_decode_varlen(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                               int B, int Hq, int Hkv, int S_max, const int32_t* cache_lens, int max_cache_len,
                               int D, attn_strides sq, attn_strides skc, attn_strides svc, attn_strides so,
                               float scale, attn_dtype dtype, int num_splits,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (!cache_lens) return ATTN_ERR_NULL;
  return decode_impl(q, k_cache, v_cache, o, lse, B, Hq, Hkv, S_max, max_cache_len, cache_lens, D, sq, skc, svc,
                     so, scale, dtype, num_splits, workspace, workspace_bytes, stream);
}

namespace {

// log2 of a supported page size (a power of two, 16 .. 2^20), else -1
static int page_log2(int page_size) {
  if (page_size < 16 || page_size > (1 << 20) || (page_size & (page_size - 1)) != 0) return -1;
  int lg = 0;
  while ((1 << lg) < page_size) ++lg;
  return lg;
}

}  // namespace

attn_status attn_decode_paged(const void* q, const void* k_pages, const void* v_pages, void* o, float* lse,
                              int B, int Hq, int Hkv, int num_pages, int page_size,
                              const int32_t* block_table, int max_pages_per_seq,
                              const int32_t* cache_lens, int max_cache_len, int D,
                              attn_strides sq, attn_strides skp, attn_strides svp, attn_strides so,
                              float scale, attn_dtype dtype, int num_splits,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (!block_table || !cache_lens) return ATTN_ERR_NULL;
  if (num_pages <= 0 || max_pages_per_seq <= 0 || max_cache_len <= 0) return ATTN_ERR_SHAPE;
  const int lg = page_log2(page_size);
  if (lg < 0) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)max_cache_len > (int64_t)max_pages_per_seq * page_size) return ATTN_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(block_table) & 3u) return ATTN_ERR_UNSUPPORTED;
  const PagedSpec pg{block_table, max_pages_per_seq, lg, num_pages};
  return decode_impl(q, k_pages, v_pages, o, lse, B, Hq, Hkv, max_cache_len, max_cache_len, cache_lens, D, sq, skp,
                     svp, so, scale, dtype, num_splits, workspace, workspace_bytes, stream, &pg);
}

attn_status attn_decode_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int Hq, int Hkv, int S_max, int cache_len, int D,
                           attn_strides sq, attn_strides sk, attn_strides sv, attn_strides so,
                           float scale, attn_dtype dtype, int num_splits, const attn_decode_opts* opts,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (!opts) return ATTN_ERR_NULL;
  if (opts->block_table) {
    if (!opts->cache_lens) return ATTN_ERR_NULL;
    if (opts->num_pages <= 0 || opts->max_pages_per_seq <= 0 || cache_len <= 0) return ATTN_ERR_SHAPE;
    const int lg = page_log2(opts->page_size);
    if (lg < 0) return ATTN_ERR_UNSUPPORTED;
    if ((int64_t)cache_len > (int64_t)opts->max_pages_per_seq * opts->page_size) return ATTN_ERR_SHAPE;
    if (reinterpret_cast<uintptr_t>(opts->block_table) & 3u) return ATTN_ERR_UNSUPPORTED;
    const PagedSpec pg{opts->block_table, opts->max_pages_per_seq, lg, opts->num_pages};
    return decode_impl(q, k, v, o, lse, B, Hq, Hkv, cache_len, cache_len, opts->cache_lens, D, sq, sk, sv, so,
                       scale, dtype, num_splits, workspace, workspace_bytes, stream, &pg, opts->window_left);
  }
  return decode_impl(q, k, v, o, lse, B, Hq, Hkv, S_max, cache_len, opts->cache_lens, D, sq, sk, sv, so, scale,
                     dtype, num_splits, workspace, workspace_bytes, stream, nullptr, opts->window_left);
}

attn_status kv_cache_write_paged(void* k_pages, void* v_pages, const void* k_new, const void* v_new,
                                 int B, int Hkv, int num_pages, int page_size, const int32_t* block_table,
                                 int max_pages_per_seq, const int32_t* pos, int D, int T,
                                 attn_strides skp, attn_strides svp, attn_strides skn, attn_strides svn,
                                 attn_dtype dtype, void* stream) {
  if (!k_pages || !v_pages || !k_new || !v_new || !block_table || !pos) return ATTN_ERR_NULL;
  if (B <= 0 || Hkv <= 0 || num_pages <= 0 || max_pages_per_seq <= 0 || D <= 0 || T <= 0) return ATTN_ERR_SHAPE;
  const int lg = page_log2(page_size);
  if (lg < 0 || D % 8 != 0 || !dtype_ok(dtype)) return ATTN_ERR_UNSUPPORTED;
  if (!strides_ok(skp) || !strides_ok(svp) || !strides_ok(skn) || !strides_ok(svn)) return ATTN_ERR_UNSUPPORTED;
  if (!writes_once({{num_pages, skp.b}, {Hkv, skp.h}, {page_size, skp.n}, {D, 1}}) ||
      !writes_once({{num_pages, svp.b}, {Hkv, svp.h}, {page_size, svp.n}, {D, 1}}))
    return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(k_pages) || !aligned16(v_pages) || !aligned16(k_new) || !aligned16(v_new))
    return ATTN_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(block_table) & 3u) || (reinterpret_cast<uintptr_t>(pos) & 3u))
    return ATTN_ERR_UNSUPPORTED;

  attn::CacheWritePagedArgs a{};
  a.kp = static_cast<uint16_t*>(k_pages);
  a.vp = static_cast<uint16_t*>(v_pages);
  a.kn = static_cast<const uint16_t*>(k_new);
  a.vn = static_cast<const uint16_t*>(v_new);
  a.block_table = block_table;
  a.pos = pos;
  a.skpp = skp.b; a.skph = skp.h; a.skpn = skp.n;
  a.svpp = svp.b; a.svph = svp.h; a.svpn = svp.n;
  a.sknb = skn.b; a.sknh = skn.h; a.sknn = skn.n;
  a.svnb = svn.b; a.svnh = svn.h; a.svnn = svn.n;
  a.rows = (int64_t)B * Hkv * T;
  a.B = B; a.Hkv = Hkv; a.T = T; a.D = D;
  a.mbps = max_pages_per_seq; a.lg_ps = lg; a.num_pages = num_pages;
  const hipError_t e = attn::launch_cache_write_paged(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

size_t attn_bwd_workspace_bytes(int B, int Hq, int Nq) {
  if (B <= 0 || Hq <= 0 || Nq <= 0) return 0;
  return (size_t)B * Hq * Nq * 8;
}

static attn_status bwd_impl(const void* q, const void* k, const void* v, const void* o, const void* dout,
                            const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq, int Nkv,
                            int D, attn_strides sq, attn_strides sk, attn_strides sv, attn_strides so,
                            attn_strides sdo, attn_strides sdq, attn_strides sdk, attn_strides sdv, float scale,
                            MaskSpec mk, attn_dtype dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return ATTN_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nkv <= 0 || D <= 0) return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if (!dtype_ok(dtype) || !std::isfinite(scale)) return ATTN_ERR_UNSUPPORTED;
  if (mk.mode < 0) return ATTN_ERR_UNSUPPORTED;
  mk = open_wide_sides(mk, Nq > Nkv ? Nq : Nkv);
  if (mk.mode == 2 && (Nq > kMaxBandRows || Nkv > kMaxBandRows)) return ATTN_ERR_UNSUPPORTED;
  for (const attn_strides* st : {&sq, &sk, &sv, &so, &sdo, &sdq, &sdk, &sdv})
    if (!strides_ok(*st) || st->n > kMaxRowStride) return ATTN_ERR_UNSUPPORTED;
  if (!writes_once({{B, sdq.b}, {Hq, sdq.h}, {Nq, sdq.n}, {D, 1}}) ||
      !writes_once({{B, sdk.b}, {Hkv, sdk.h}, {Nkv, sdk.n}, {D, 1}}) ||
      !writes_once({{B, sdv.b}, {Hkv, sdv.h}, {Nkv, sdv.n}, {D, 1}}))
    return ATTN_ERR_UNSUPPORTED;
  for (const void* p : {q, k, v, o, dout, static_cast<const void*>(dq), static_cast<const void*>(dk),
                        static_cast<const void*>(dv)})
    if (!aligned16(p)) return ATTN_ERR_UNSUPPORTED;
  if (reinterpret_cast<uintptr_t>(lse) & 3u) return ATTN_ERR_UNSUPPORTED;
  const size_t need = attn_bwd_workspace_bytes(B, Hq, Nq);
  if (!workspace || !aligned16(workspace) || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  const int64_t nqb = ((int64_t)Nq + 255) / 256;   // dq: 256 query rows per workgroup
  const int64_t nkb = ((int64_t)Nkv + 127) / 128;  // dkdv: 128 keys per workgroup
  const int64_t dq_blocks = nqb * Hq * B, dkv_blocks = nkb * Hkv * B;
  if (dq_blocks > INT_MAX || dkv_blocks > INT_MAX || (int64_t)B * Hq * Nq > INT_MAX) return ATTN_ERR_SHAPE;

  attn::BwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(o);
  a.dout = static_cast<const uint16_t*>(dout);
  a.lse = lse;
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.ld = static_cast<float*>(workspace);
  a.sqb = sq.b; a.sqh = sq.h; a.sqn = sq.n;
  a.skb = sk.b; a.skh = sk.h; a.skn = sk.n;
  a.svb = sv.b; a.svh = sv.h; a.svn = sv.n;
  a.sob = so.b; a.soh = so.h; a.son = so.n;
  a.sdob = sdo.b; a.sdoh = sdo.h; a.sdon = sdo.n;
  a.sdqb = sdq.b; a.sdqh = sdq.h; a.sdqn = sdq.n;
  a.sdkb = sdk.b; a.sdkh = sdk.h; a.sdkn = sdk.n;
  a.sdvb = sdv.b; a.sdvh = sdv.h; a.sdvn = sdv.n;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Nq = Nq; a.Nkv = Nkv; a.group = Hq / Hkv;
  a.nqb = (int)nqb;
  a.nkb = (int)nkb;
  a.dq_blocks = (unsigned)dq_blocks;
  a.dkv_blocks = (unsigned)dkv_blocks;
  // XCD-aware block order, as the forward's: workgroup i runs on XCD i % 8,
  // and the remap gives each XCD a contiguous span of whole (batch, kv head)
  // units, so the workgroups that stream one kv head's K and V (dQ pass) or
  // its q heads' Q and dO rows (dK/dV pass) run on one XCD and meet in its L2
  a.dq_remap = (dq_blocks % 8 == 0) && (dq_blocks / 8) % ((int64_t)a.group * nqb) == 0;
  a.dkv_remap = (dkv_blocks % 8 == 0) && (dkv_blocks / 8) % nkb == 0;
  a.mask = mk.mode;
  a.causal_off = mk.bottom_right ? Nkv - Nq : 0;
  a.win_left = mk.left;
  a.win_right = mk.right;
  a.bf16 = dtype == ATTN_BF16;
  a.c = scale * kLog2e;
  a.scale = scale;
  a.q_bytes = slice_bytes(Nq, sq.n, D);
  a.k_bytes = slice_bytes(Nkv, sk.n, D);
  a.v_bytes = slice_bytes(Nkv, sv.n, D);
  a.do_bytes = slice_bytes(Nq, sdo.n, D);
  const hipError_t e = attn::launch_bwd(a, D, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

static attn_status bwd_varlen_impl(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                   const float* lse, void* dq, void* dk, void* dv, const int32_t* cu_seqlens_q,
                                   const int32_t* cu_seqlens_k, int B, int max_seqlen_q, int max_seqlen_k,
                                   int total_q, int total_k, int Hq, int Hkv, int D, attn_strides sq,
                                   attn_strides sk, attn_strides sv, attn_strides so, attn_strides sdo,
                                   attn_strides sdq, attn_strides sdk, attn_strides sdv, float scale, MaskSpec mk,
                                   attn_dtype dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !cu_seqlens_q || !cu_seqlens_k)
    return ATTN_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || max_seqlen_q <= 0 || max_seqlen_k <= 0 || total_q <= 0 || total_k < 0 ||
      D <= 0)
    return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if (!dtype_ok(dtype) || !std::isfinite(scale)) return ATTN_ERR_UNSUPPORTED;
  if (mk.mode < 0) return ATTN_ERR_UNSUPPORTED;
  mk = open_wide_sides(mk, total_q > total_k ? total_q : total_k);
  if (mk.mode == 2 && (total_q > kMaxBandRows || total_k > kMaxBandRows)) return ATTN_ERR_UNSUPPORTED;
  // packed (token, head, dim) views: the batch stride is unused and not checked
  for (attn_strides* st : {&sq, &sk, &sv, &so, &sdo, &sdq, &sdk, &sdv}) {
    st->b = 0;
    if (!strides_ok(*st) || st->n > kMaxRowStride) return ATTN_ERR_UNSUPPORTED;
  }
  if (!writes_once({{total_q, sdq.n}, {Hq, sdq.h}, {D, 1}}) || !writes_once({{total_k, sdk.n}, {Hkv, sdk.h}, {D, 1}}) ||
      !writes_once({{total_k, sdv.n}, {Hkv, sdv.h}, {D, 1}}))
    return ATTN_ERR_UNSUPPORTED;
  for (const void* p : {q, k, v, o, dout, static_cast<const void*>(dq), static_cast<const void*>(dk),
                        static_cast<const void*>(dv)})
    if (!aligned16(p)) return ATTN_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(lse) & 3u) || (reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3u) ||
      (reinterpret_cast<uintptr_t>(cu_seqlens_k) & 3u))
    return ATTN_ERR_UNSUPPORTED;
  const size_t need = attn_bwd_workspace_bytes(1, Hq, total_q);
  if (!workspace || !aligned16(workspace) || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  const int64_t nqb = ((int64_t)max_seqlen_q + 255) / 256;
  const int64_t nkb = ((int64_t)max_seqlen_k + 127) / 128;
  const int64_t dq_blocks = nqb * Hq * B, dkv_blocks = nkb * Hkv * B;
  if (dq_blocks > INT_MAX || dkv_blocks > INT_MAX || (int64_t)Hq * total_q > INT_MAX) return ATTN_ERR_SHAPE;

  attn::BwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(o);
  a.dout = static_cast<const uint16_t*>(dout);
  a.lse = lse;
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.ld = static_cast<float*>(workspace);
  a.sqh = sq.h; a.sqn = sq.n;
  a.skh = sk.h; a.skn = sk.n;
  a.svh = sv.h; a.svn = sv.n;
  a.soh = so.h; a.son = so.n;
  a.sdoh = sdo.h; a.sdon = sdo.n;
  a.sdqh = sdq.h; a.sdqn = sdq.n;
  a.sdkh = sdk.h; a.sdkn = sdk.n;
  a.sdvh = sdv.h; a.sdvn = sdv.n;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.group = Hq / Hkv;
  a.Nq = max_seqlen_q;   // per-sequence rows are capped at these bounds
  a.Nkv = max_seqlen_k;
  a.nqb = (int)nqb;
  a.nkb = (int)nkb;
  a.dq_blocks = (unsigned)dq_blocks;
  a.dkv_blocks = (unsigned)dkv_blocks;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.total_q = total_q;
  a.total_k = total_k;
  a.causal_br = mk.bottom_right;
  a.mask = mk.mode;
  a.win_left = mk.left;
  a.win_right = mk.right;
  a.bf16 = dtype == ATTN_BF16;
  a.c = scale * kLog2e;
  a.scale = scale;
  const hipError_t e = attn::launch_bwd(a, D, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const void* dout,
                            const float* lse, void* dq, void* dk, void* dv, const int32_t* cu_seqlens_q,
                            const int32_t* cu_seqlens_k, int B, int max_seqlen_q, int max_seqlen_k, int total_q,
                            int total_k, int Hq, int Hkv, int D, attn_strides sq, attn_strides sk, attn_strides sv,
                            attn_strides so, attn_strides sdo, attn_strides sdq, attn_strides sdk, attn_strides sdv,
                            float scale, int causal, attn_dtype dtype, void* workspace, size_t workspace_bytes,
                            void* stream) {
  return bwd_varlen_impl(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, B, max_seqlen_q,
                         max_seqlen_k, total_q, total_k, Hq, Hkv, D, sq, sk, sv, so, sdo, sdq, sdk, sdv, scale,
                         mask_of_causal(causal), dtype, workspace, workspace_bytes, stream);
}

attn_status attn_bwd_varlen_masked(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                   const float* lse, void* dq, void* dk, void* dv, const int32_t* cu_seqlens_q,
                                   const int32_t* cu_seqlens_k, int B, int max_seqlen_q, int max_seqlen_k,
                                   int total_q, int total_k, int Hq, int Hkv, int D, attn_strides sq,
                                   attn_strides sk, attn_strides sv, attn_strides so, attn_strides sdo,
                                   attn_strides sdq, attn_strides sdk, attn_strides sdv, float scale,
                                   attn_mask mask, attn_dtype dtype, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  return bwd_varlen_impl(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, B, max_seqlen_q,
                         max_seqlen_k, total_q, total_k, Hq, Hkv, D, sq, sk, sv, so, sdo, sdq, sdk, sdv, scale,
                         mask_of(mask), dtype, workspace, workspace_bytes, stream);
}

attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                     void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq, int Nkv, int D,
                     attn_strides sq, attn_strides sk, attn_strides sv, attn_strides so, attn_strides sdo,
                     attn_strides sdq, attn_strides sdk, attn_strides sdv, float scale, int causal,
                     attn_dtype dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, D, sq, sk, sv, so, sdo, sdq, sdk, sdv,
                  scale, mask_of_causal(causal), dtype, workspace, workspace_bytes, stream);
}

attn_status attn_bwd_masked(const void* q, const void* k, const void* v, const void* o, const void* dout,
                            const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq, int Nkv,
                            int D, attn_strides sq, attn_strides sk, attn_strides sv, attn_strides so,
                            attn_strides sdo, attn_strides sdq, attn_strides sdk, attn_strides sdv, float scale,
                            attn_mask mask, attn_dtype dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, D, sq, sk, sv, so, sdo, sdq, sdk, sdv,
                  scale, mask_of(mask), dtype, workspace, workspace_bytes, stream);
}

attn_status kv_cache_write(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                           int B, int Hkv, int S_max, int D, int pos, int T,
                           attn_strides skc, attn_strides svc, attn_strides skn, attn_strides svn,
                           attn_dtype dtype, void* stream) {
  if (!k_cache || !v_cache || !k_new || !v_new) return ATTN_ERR_NULL;
  if (B <= 0 || Hkv <= 0 || S_max <= 0 || D <= 0 || T <= 0) return ATTN_ERR_SHAPE;
  if (pos < 0 || (int64_t)pos + T > S_max) return ATTN_ERR_SHAPE;
  if (D % 8 != 0 || !dtype_ok(dtype)) return ATTN_ERR_UNSUPPORTED;
  if (!strides_ok(skc) || !strides_ok(svc) || !strides_ok(skn) || !strides_ok(svn)) return ATTN_ERR_UNSUPPORTED;
  if (!writes_once({{B, skc.b}, {Hkv, skc.h}, {S_max, skc.n}, {D, 1}}) ||
      !writes_once({{B, svc.b}, {Hkv, svc.h}, {S_max, svc.n}, {D, 1}}))
    return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new))
    return ATTN_ERR_UNSUPPORTED;

  attn::CacheWriteArgs a{};
  a.kc = static_cast<uint16_t*>(k_cache);
  a.vc = static_cast<uint16_t*>(v_cache);
  a.kn = static_cast<const uint16_t*>(k_new);
  a.vn = static_cast<const uint16_t*>(v_new);
  a.skcb = skc.b; a.skch = skc.h; a.skcn = skc.n;
  a.svcb = svc.b; a.svch = svc.h; a.svcn = svc.n;
  a.sknb = skn.b; a.sknh = skn.h; a.sknn = skn.n;
  a.svnb = svn.b; a.svnh = svn.h; a.svnn = svn.n;
  a.Hkv = Hkv; a.pos = pos; a.T = T; a.D = D;
  a.rows = (int64_t)B * Hkv * T;
  const hipError_t e = attn::launch_cache_write(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // extern "C"
