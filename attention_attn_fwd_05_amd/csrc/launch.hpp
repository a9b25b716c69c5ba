// Host-visible argument blocks and launchers of the attention kernels.  The C
// ABI layer (attn_api.cpp) validates arguments and fills these; each launcher
// enqueues its kernels on the given stream and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;  // nullable, contiguous (B, Hq, Nq)
  int64_t sqb, sqh, sqn;
  int64_t skb, skh, skn;
  int64_t svb, svh, svn;
  int64_t sob, soh, son;
  int Hq, Hkv, Nq, Nkv, group;
  int nqb;      // number of query blocks (rows per workgroup: see the kernel)
  int nblocks;  // grid size
  int remap;    // 1: XCD-aware block remap is valid for this grid
  int causal_off;  // causal: query i sees keys j <= i + causal_off
  float c;      // |scale| * log2(e), or a tiny positive value when scale == 0
  uint32_t qsign;  // 0x80008000 when scale < 0: flip Q's sign bits (exact)
  // bytes from a (batch, head) slice's first element to the end of its last
  // valid row: buffer loads at or past this offset read zeros
  int64_t q_bytes, k_bytes, v_bytes;
  // packed variable-length batches (null otherwise): sequence b owns query
  // rows [cu_q[b], cu_q[b+1]) of total_q and key rows [cu_k[b], cu_k[b+1]) of
  // total_k; lse is then (Hq, total_q)
  const int32_t* cu_q;
  const int32_t* cu_k;
  int total_q, total_k;
  int units;      // B * Hkv
  int causal_br;  // causal offset per sequence: 1 = L_k - L_q, 0 = 0
  // band mask (mask mode 2): query i sees keys i + off - win_left <= j <=
  // i + off + win_right; -1 leaves that side open
  int win_left, win_right;
  int rows;  // query rows per workgroup: 256; 128 for dense grids that 256-row blocks leave half empty and for packed batches of short sequences
  int ring_polls;  // masked grids' counted KV ring: polls a wait makes before it gives up
};

// mask: 0 none, 1 causal, 2 band
hipError_t launch_prefill(const FwdArgs& a, int D, bool bf16, int mask, bool varlen, hipStream_t stream);

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;  // nullable, contiguous (B, Hq)
  const int32_t* lens;  // nullable: per-sequence lengths, clamped to [0, cache_len]
  int64_t sqb, sqh;
  int64_t skb, skh, skn;
  int64_t svb, svh, svn;
  int64_t sob, soh;
  int Hq, Hkv, group, cache_len;  // cache_len: every sequence's length, or the bound on lens
  int heads_per_wg;  // q heads handled by one workgroup (<= 16)
  int hgroups;       // head groups per kv head
  int nsplit;          // chunks along the cache (<= max_splits)
  int max_splits;      // partial slots per (unit, head group) in the workspace (<= 64)
  int rows_per_split;  // multiple of the 128-row tile
  int unit_fast;       // grid order: 1 = (unit, head group, chunk), 0 = (chunk, head group, unit)
  float c;
  uint32_t qsign;
  float* part;  // workspace: partial (m, l, pad, pad, o[D]) per (unit, head group, split, head)
  // paged cache (null otherwise): slot r of sequence b is row r & (2^lg_ps - 1)
  // of page block_table[b * mbps + (r >> lg_ps)]; k / v then point at page 0
  // and skb / svb are the page strides
  const int32_t* block_table;
  int mbps, lg_ps, num_pages;
  // sliding window: -1 none; w >= 0 keeps slots >= len - 1 - w (the query is
  // the last slot); chunks then start at the 128-slot tile holding that slot
  int window_left;
};

hipError_t launch_decode(const DecodeArgs& a, int B, int D, bool bf16, hipStream_t stream);

// Device address of the library's own decode scratch (ATTN_DECODE_NOALLOC_SCRATCH_BYTES
// bytes) on the device `stream` runs on (the current device for a null stream),
// looked up once per device and kept.  Allocates nothing.
hipError_t decode_scratch_address(hipStream_t stream, void** addr);

struct CacheWritePagedArgs {
  uint16_t* kp;
  uint16_t* vp;
  const uint16_t* kn;
  const uint16_t* vn;
  const int32_t* block_table;
  const int32_t* pos;  // per sequence: slot of its first new row
  int64_t skpp, skph, skpn;  // page pool strides (page, head, row)
  int64_t svpp, svph, svpn;
  int64_t sknb, sknh, sknn;
  int64_t svnb, svnh, svnn;
  int64_t rows;  // B * Hkv * T
  int B, Hkv, T, D, mbps, lg_ps, num_pages;
};

hipError_t launch_cache_write_paged(const CacheWritePagedArgs& a, hipStream_t stream);

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;  // contiguous (B, Hq, Nq), natural log, from the forward
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* ld;  // workspace: (lse * log2 e, delta) per query row, (B, Hq, Nq, 2)
  int64_t sqb, sqh, sqn;
  int64_t skb, skh, skn;
  int64_t svb, svh, svn;
  int64_t sob, soh, son;
  int64_t sdob, sdoh, sdon;
  int64_t sdqb, sdqh, sdqn;
  int64_t sdkb, sdkh, sdkn;
  int64_t sdvb, sdvh, sdvn;
  int B, Hq, Hkv, Nq, Nkv, group;
  int nqb, nkb;                // query blocks (dq), key blocks (dkdv) per (batch, head)
  unsigned dq_blocks, dkv_blocks;
  // 1: XCD-aware block order (dense grids whose 8 XCD spans hold whole
  // (batch, kv head) units), for the dQ and the dK/dV pass
  int dq_remap, dkv_remap;
  // packed variable-length batches (null otherwise): sequence b owns query rows
  // [cu_q[b], cu_q[b+1]) and key rows [cu_k[b], cu_k[b+1]); B is then the
  // number of sequences, Nq / Nkv the max_seqlen bounds, and lse and the
  // workspace rows are (Hq, total_q)
  const int32_t* cu_q;
  const int32_t* cu_k;
  int total_q, total_k;
  int causal_br;               // packed: causal offset per sequence, 1 = L_k - L_q
  int mask;                    // 0 none, 1 causal, 2 band
  int causal_off;              // query i sits at key position i + causal_off
  int win_left, win_right;     // band bounds around that position (-1: open)
  int bf16;
  float c;                     // scale * log2(e)
  float scale;
  // bytes from a (batch, head) slice's first element to the end of its last row
  int64_t q_bytes, k_bytes, v_bytes, do_bytes;
};

hipError_t launch_bwd(const BwdArgs& a, int D, hipStream_t stream);

struct CacheWriteArgs {
  uint16_t* kc;
  uint16_t* vc;
  const uint16_t* kn;
  const uint16_t* vn;
  int64_t skcb, skch, skcn;
  int64_t svcb, svch, svcn;
  int64_t sknb, sknh, sknn;
  int64_t svnb, svnh, svnn;
  int Hkv, pos, T, D;
  int64_t rows;  // B * Hkv * T
};

hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t stream);

}  // namespace attn
