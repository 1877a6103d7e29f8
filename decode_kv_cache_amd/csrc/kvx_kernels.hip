// libkvx device side for gfx950 (CDNA4): the layer copy kernel behind
// kvx_push_layer / kvx_pack / kvx_unpack, the batched copy kernel behind
// kvx_push_many and multi-layer kvx_pack / kvx_unpack, and the head-slice
// kernel behind kvx_copy_heads, with their C entry points.
//
// The work is pure data movement bound by HBM bandwidth: no arithmetic, no
// MFMA.  Each workgroup owns one piece, or one 4 KiB chunk of a piece, of
// one (layer, region) pair (4 to 32 KiB, by the launch shape); every lane
// issues all of its 16-byte loads before its first store so that a
// workgroup keeps the whole piece in flight.  Piece records are
// workgroup-uniform and come in through scalar loads.
//
// Sources: [PUSH] push-based NIXL connector post, [MORI] MoRIIO connector
// note, [BIDIR] bidirectional KV transfer post (full titles in kvx.h).

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "kvx_internal.h"

namespace kvx {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

enum Mode : int { kPush = 0, kPack = 1, kUnpack = 2 };

// Maximum workgroups per launch along x; larger work lists are split.
constexpr int64_t kMaxGridX = int64_t(1) << 22;

// The chip deals a launch's workgroups to its eight XCDs round robin by
// dispatch index, and each XCD has its own L2 and address-translation
// caches.  A launch of n work items (pieces or chunks) mapped XCD-aware takes
// xcd_span(n) = 8 ceil(n / 8) workgroups along x, and workgroup x works on
// item xcd_item(x): XCD k walks the k-th contiguous eighth of the work list
// instead of every eighth item, so each XCD touches an eighth of the pages.
// Workgroups past the items exit.  Measured per layer on one MI355X, plain
// mapping against XCD-aware: 32-layer batched launches of the 536 MB-per-
// region batched table 751 -> 714 us, of the Qwen3-32B-shaped table with
// block-size change 10.83 -> 10.28 us; per-layer launches of the batched
// table 739 -> 732 us, of 32 KiB pieces 12.3 -> 12.1 us.  Launches of
// fewer than 65536 4 KiB pieces lose by it (GPT-OSS full-attention group
// 44.5 -> 45.7 us, the MLA latent pool 27.7 -> 28.2 us) and keep the plain
// mapping, as does the head-slice kernel (no gain).
constexpr int64_t kXcds = 8;
constexpr int64_t kXcdFineMin = 65536;
static bool xcd_on(bool fine, int64_t n) { return !fine || n >= kXcdFineMin; }
static int64_t xcd_span(int64_t n, bool on) { return on ? (n + kXcds - 1) / kXcds * kXcds : n; }
__device__ __forceinline__ int xcd_item(int x, int span, int on) {
  return on ? (x % int(kXcds)) * (span / int(kXcds)) + x / int(kXcds) : x;
}

struct CopyArgs {
  const Piece* pieces;       // already offset by the launch's first piece
  const BlockPair* blocks;
  int32_t n_pieces;          // pieces in this launch
  int32_t n_blocks;          // planned blocks (scale entries)
  int32_t n_scale_slots;     // scale entries to write (pack: padded to 16 B)
  int32_t first_scale_wg;    // x index of the first scale workgroup (== xcd_span(n_pieces))
  int32_t xcd;               // pieces mapped XCD-aware
  const uint8_t* in[2];      // region 0 / 1 source (pool or staging): K, V or conv, SSM
  uint8_t* out[2];           // region 0 / 1 destination (pool or staging)
  const uint32_t* in_sc[2];  // scale source (pool scales or staging scale segment)
  uint32_t* out_sc[2];
};

// Cache policy of the copies (buffer instruction aux bits on gfx950: bit 0 =
// sc0, bit 1 = nt, bit 4 = sc1).  Nothing is re-read, so loads are
// non-temporal (nt).  Stores depend on the launch shape, from side-by-side
// measurements:
//  - one-wave pieces (a launch of about one round) store nt: adding sc0 and
//    sc1 made the Qwen3-32B-shaped layer 1.8% slower;
//  - 4 KiB pieces of four-wave workgroups (streaming launches) store nt sc0
//    sc1, write-through at system scope: 2.8-4% faster on the large
//    attention layers and the batched push, and about 10% faster when a
//    compute kernel that ends in stores of its own runs beside the push
//    (each such kernel's end waits for dirty lines in L2, the push's
//    included).
#ifndef KVX_LD_AUX
#define KVX_LD_AUX 2
#endif
#ifndef KVX_ST_AUX_ONE_WAVE
#define KVX_ST_AUX_ONE_WAVE 2
#endif
#ifndef KVX_ST_AUX_FINE
#define KVX_ST_AUX_FINE 19
#endif
constexpr int kBufferWord3 = 0x00020000;  // raw byte buffer, gfx9 family

// A workgroup's piece record, read through the constant address space so
// that it arrives in scalar registers through scalar loads.  Read as an
// ordinary global load, part of it landed in vector registers; the buffer
// resources built from it were then not provably uniform and every buffer
// instruction was wrapped in a readfirstlane loop.
typedef const __attribute__((address_space(4))) v4u* ConstVecs;
struct PieceBits {
  v4u lo, hi;
};
static_assert(sizeof(PieceBits) == sizeof(Piece), "a piece record is two 16-byte vectors");
__device__ __forceinline__ Piece load_piece(const Piece* list, int i) {
  const ConstVecs q = (ConstVecs)(list + i);
  const PieceBits b = {q[0], q[1]};
  return __builtin_bit_cast(Piece, b);
}

// Region pointer r (0 or 1) of a two-entry kernel-argument array, chosen
// by a select rather than an indexed access into the argument block (the
// compiler turns it into one scalar-cache load at the selected offset).
template <typename P>
__device__ __forceinline__ P pick(P const (&a)[2], int r) { return r ? a[1] : a[0]; }

// Copy `len` bytes (a piece, at most T x V x 16) from `src` to `dst` with
// the whole workgroup of T lanes, each keeping V 16-byte vectors in flight.
// One buffer resource per piece (base = piece start, size = piece length):
// lanes past a short piece's end read zeros and their stores are dropped by
// the hardware range check, so every lane issues all of its loads before its
// first store without any masking.
template <int T, int V>
__device__ __forceinline__ void copy_piece(const uint8_t* src, uint8_t* dst, int32_t len) {
  constexpr int kStAux = T == 64 ? KVX_ST_AUX_ONE_WAVE : KVX_ST_AUX_FINE;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src), (short)0, len, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(dst, (short)0, len, kBufferWord3);
  const int t = threadIdx.x;
  v4u r[V];
#pragma unroll
  for (int k = 0; k < V; ++k)
    r[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, (t + k * T) * 16, 0, KVX_LD_AUX);
#pragma unroll
  for (int k = 0; k < V; ++k)
    __builtin_amdgcn_raw_buffer_store_b128(r[k], rd, (t + k * T) * 16, 0, kStAux);
}

// One workgroup copies one piece of region blockIdx.y + piece.reg (one list
// shared by K and V: y picks the region; one list per region: the tag does);
// workgroups past the pieces copy the planned blocks' scales, one per lane.
template <int MODE, int T, int V>
__global__ __launch_bounds__(T) void copy_kernel(CopyArgs a) {
  const int x = blockIdx.x;
  if (x < a.first_scale_wg) {
    const int i = xcd_item(x, a.first_scale_wg, a.xcd);
    if (i >= a.n_pieces) return;
    const Piece pc = load_piece(a.pieces, i);
    const int kv = int(blockIdx.y) + pc.reg;
    const int64_t ioff = MODE == kUnpack ? pc.stg_off : pc.src_off;
    const int64_t ooff = MODE == kPack ? pc.stg_off : pc.dst_off;
    copy_piece<T, V>(pick(a.in, kv) + ioff, pick(a.out, kv) + ooff, pc.len);
    return;
  }
  const int kv = blockIdx.y;
  const int i = (x - a.first_scale_wg) * T + threadIdx.x;
  if (MODE == kPush) {
    if (i < a.n_blocks) {
      const BlockPair b = a.blocks[i];
      a.out_sc[kv][b.dst] = a.in_sc[kv][b.src];
    }
  } else if (MODE == kPack) {
    if (i < a.n_blocks)
      a.out_sc[kv][i] = a.in_sc[kv][a.blocks[i].src];
    else if (i < a.n_scale_slots)
      a.out_sc[kv][i] = 0u;
  } else {
    if (i < a.n_blocks) a.out_sc[kv][a.blocks[i].dst] = a.in_sc[kv][i];
  }
}

struct RunArgs {
  const RunRec* runs;        // run table of the mode's order
  const uint32_t* gidx;      // first run of each group of kRunGroupChunks chunks
  const BlockPair* blocks;
  uint32_t nruns, total16;   // runs; flat length in 16-byte units
  int32_t n_chunks;          // 4 KiB chunks
  int32_t chunk_span;        // xcd_span(n_chunks): workgroups before the scale workgroups
  int32_t xcd;               // chunks mapped XCD-aware
  int32_t n_blocks, n_scale_slots;
  uint32_t in_bytes, out_bytes;  // bytes addressable from in[r] / out[r]
  const uint8_t* in[2];
  uint8_t* out[2];
  const uint32_t* in_sc[2];
  uint32_t* out_sc[2];
};

// One workgroup copies one 4 KiB chunk of a run table's flat space (the
// runs back to back in the table's order) of region blockIdx.y.  Each wave
// covers 64 consecutive 16-byte units.  Starting from the first run of the
// chunk's group (a run index entry per kRunGroupChunks chunks), the wave
// walks the run records with scalar loads: past the runs that end before its
// first unit, then over the runs that start inside its 64 units, each lane
// keeping the last one that starts at or before its unit.  Long runs make
// this one or two record loads per wave.  No per-piece record exists: the
// work list is the run table, 16 bytes per run, plus its run index.
// Addresses are 32-bit byte offsets into one buffer resource per region.
// Workgroups past the chunks copy the planned blocks' scales, as in
// copy_kernel.
typedef const __attribute__((address_space(4))) uint32_t* ConstU32;
__device__ __forceinline__ RunRec load_run(const RunRec* t, uint32_t i) {
  return __builtin_bit_cast(RunRec, ((ConstVecs)t)[i]);
}
template <int MODE>
__global__ __launch_bounds__(256) void run_kernel(RunArgs a) {
  const int xw = blockIdx.x;
  const int kv = blockIdx.y;
  if (xw < a.chunk_span) {
    const int x = xcd_item(xw, a.chunk_span, a.xcd);
    if (x >= a.n_chunks) return;
    const uint32_t lane = threadIdx.x & 63u;
    // the wave's first unit, made visibly wave-uniform so that the record
    // walk below stays in scalar registers
    const uint32_t fw = __builtin_amdgcn_readfirstlane(uint32_t(x) * uint32_t(kRunChunk16) + (threadIdx.x >> 6) * 64u);
    if (fw >= a.total16) return;
    const uint32_t fl = fw + lane;
    const bool live = fl < a.total16;
    const uint32_t wend = min(fw + 64u, a.total16);
    uint32_t r = ((ConstU32)a.gidx)[uint32_t(x) / uint32_t(kRunGroupChunks)];
    RunRec rec = load_run(a.runs, r);
    // the run holding the wave's first unit (runs tile the flat space, so
    // this ends within the table)
    while (rec.start16 + rec.len16 <= fw && r + 1 < a.nruns) rec = load_run(a.runs, ++r);
    uint32_t my_src = rec.src16, my_dst = rec.dst16, my_start = rec.start16;
    uint32_t end = rec.start16 + rec.len16;
    // the runs that start inside the wave's units
    while (end < wend && r + 1 < a.nruns) {
      rec = load_run(a.runs, ++r);
      if (fl >= rec.start16) {
        my_src = rec.src16;
        my_dst = rec.dst16;
        my_start = rec.start16;
      }
      end = rec.start16 + rec.len16;
    }
    const bool found = fl >= my_start;
    if (!live || !found) return;
    const uint32_t d = fl - my_start;
    const uint32_t ioff = MODE == kUnpack ? fl * 16u : (my_src + d) * 16u;
    const uint32_t ooff = MODE == kPack ? fl * 16u : (my_dst + d) * 16u;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(pick(a.in, kv)), (short)0, int(a.in_bytes), kBufferWord3);
    const __amdgpu_buffer_rsrc_t rd =
        __builtin_amdgcn_make_buffer_rsrc(pick(a.out, kv), (short)0, int(a.out_bytes), kBufferWord3);
    const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rs, int(ioff), 0, KVX_LD_AUX);
    __builtin_amdgcn_raw_buffer_store_b128(v, rd, int(ooff), 0, KVX_ST_AUX_FINE);
    return;
  }
  const int i = (xw - a.chunk_span) * 256 + threadIdx.x;
  if (MODE == kPush) {
    if (i < a.n_blocks) {
      const BlockPair b = a.blocks[i];
      a.out_sc[kv][b.dst] = a.in_sc[kv][b.src];
    }
  } else if (MODE == kPack) {
    if (i < a.n_blocks)
      a.out_sc[kv][i] = a.in_sc[kv][a.blocks[i].src];
    else if (i < a.n_scale_slots)
      a.out_sc[kv][i] = 0u;
  } else {
    if (i < a.n_blocks) a.out_sc[kv][a.blocks[i].dst] = a.in_sc[kv][i];
  }
}

// Several (plan, layer) copies of one mode in one launch (kvx_push_many;
// kvx_pack / kvx_unpack over several layers): entry j owns workgroups
// [first_j, first_{j+1}) and copies its plan's pieces between its region
// bases (pool regions of its layer, or that layer's staging segments), each
// piece as 2^shift_j chunks of T x V x 16 bytes (one workgroup per chunk),
// so plans cut into larger pieces can run in a smaller launch shape without
// re-cutting their work lists.
constexpr int kManyMax = 32;
struct ManyEntry {
  const Piece* pieces;
  const uint8_t* in[2];
  uint8_t* out[2];
  int32_t first;  // x index of the entry's first workgroup
  int32_t shift;  // log2 of workgroups per piece
};
struct ManyArgs {
  int32_t n;        // entries
  int32_t items;    // workgroups' worth of work (chunks of every entry)
  int32_t span;     // xcd_span(items): workgroups along x
  int32_t xcd;      // workgroups mapped XCD-aware
  int32_t uniform;  // every entry's workgroup count when they are all alike, else 0
  int32_t pad[3];
  ManyEntry e[kManyMax];
};

template <int MODE, int T, int V>
__global__ __launch_bounds__(T) void copy_many_kernel(ManyArgs a) {
  const int x = xcd_item(blockIdx.x, a.span, a.xcd);
  if (x >= a.items) return;
  // The last entry whose first workgroup is <= x: a division when every
  // entry has the same workgroup count (several layers of one plan: the
  // queue's groups, multi-layer pack and unpack), else a binary search with
  // scalar loads.  Side by side against the search alone: the Qwen3-32B-
  // shaped queue step 6399 -> 6453 GB/s, 32 MLA latent layers per launch
  // 25.7 -> 24.7 us per layer; a linear count over all 32 entries' first
  // workgroups was no faster than the search.
  int lo = 0, hi = a.n - 1;
  if (a.uniform) {
    lo = x / a.uniform;
  } else {
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.e[mid].first <= x)
        lo = mid;
      else
        hi = mid - 1;
    }
  }
  const ManyEntry& en = a.e[lo];
  const int local = x - en.first;
  const Piece pc = load_piece(en.pieces, local >> en.shift);
  const int32_t off = (local & ((1 << en.shift) - 1)) * (T * V * 16);
  const int32_t len = std::min(pc.len - off, T * V * 16);
  if (len <= 0) return;  // a chunk past the end of a short piece
  const int kv = int(blockIdx.y) + pc.reg;
  const int64_t ioff = MODE == kUnpack ? pc.stg_off : pc.src_off;
  const int64_t ooff = MODE == kPack ? pc.stg_off : pc.dst_off;
  copy_piece<T, V>(pick(en.in, kv) + ioff + off, pick(en.out, kv) + ooff + off, len);
}

// The per-block scale copies of several (plan, layer) entries of one mode in
// one launch: the scale workgroups of copy_kernel, batched like
// copy_many_kernel.  Entry j owns workgroups [first_j, first_{j+1}), one
// lane per scale entry, and region blockIdx.y.
struct ScaleEntry {
  const BlockPair* blocks;
  const uint32_t* in_sc[2];
  uint32_t* out_sc[2];
  int32_t n_blocks;  // planned blocks
  int32_t n_slots;   // scale entries to write (pack: padded to 16 B)
  int32_t first;     // x index of the entry's first workgroup
  int32_t pad;
};
struct ScaleManyArgs {
  int32_t n;  // entries
  int32_t pad[3];
  ScaleEntry e[kManyMax];
};
constexpr int kScaleThreads = 256;

template <int MODE>
__global__ __launch_bounds__(kScaleThreads) void scale_many_kernel(ScaleManyArgs a) {
  const int x = blockIdx.x;
  const int kv = blockIdx.y;
  int lo = 0, hi = a.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.e[mid].first <= x)
      lo = mid;
    else
      hi = mid - 1;
  }
  const ScaleEntry& en = a.e[lo];
  const int i = (x - en.first) * kScaleThreads + int(threadIdx.x);
  if (MODE == kPush) {
    if (i < en.n_blocks) {
      const BlockPair b = en.blocks[i];
      en.out_sc[kv][b.dst] = en.in_sc[kv][b.src];
    }
  } else if (MODE == kPack) {
    if (i < en.n_blocks)
      en.out_sc[kv][i] = en.in_sc[kv][en.blocks[i].src];
    else if (i < en.n_slots)
      en.out_sc[kv][i] = 0u;
  } else {
    if (i < en.n_blocks) en.out_sc[kv][en.blocks[i].dst] = en.in_sc[kv][i];
  }
}

struct HeadArgs {
  const BlockPair* blocks;   // already offset by the launch's first block
  const uint8_t* in[2];
  uint8_t* out[2];
  const uint32_t* in_sc[2];  // NULL without scales
  uint32_t* out_sc[2];
  int64_t s_blk, s_slot, s_head;  // source byte strides
  int64_t d_blk, d_slot, d_head;  // destination byte strides
  int32_t vpr;                    // 16-B vectors per (token, head) row
  int32_t nh;                     // heads in the slice
  int32_t dst_head_major;         // 1: enumerate (head, slot, vec) -- HND destination

};

// Store policy of heads_kernel: the streaming copies' write-through nt sc0
// sc1 (side by side with nt alone on the TP4 head slice: 53.1 against 53.3
// us per layer, no real difference; this kernel is bound by its strided
// source rows).
#ifndef KVX_HEAD_ST_AUX
#define KVX_HEAD_ST_AUX KVX_ST_AUX_FINE
#endif
// 512 lanes: on the TP4 head share (8 KiB per block, 512 vectors) every
// lane moves one vector.  Side by side, us per layer: 512 lanes 49.3-49.8,
// 256 lanes 50.2-51.5, 128 lanes 50.9-52.0; a workgroup taking two or four
// planned blocks with all their loads ahead of the stores 51.9 and 52.2
// against 49.6; launches allowed to overlap the previous one on the stream
// made no consistent difference.
constexpr int kHeadThreads = 512;
constexpr int kHeadUnroll = 4;

// One workgroup moves the head slice of one planned block (or block piece,
// with different block sizes per side) of region blockIdx.y (K, V or the
// latent region).  Lanes walk the block's rows in destination order so
// stores are contiguous; each lane keeps kHeadUnroll vectors in flight.
__device__ __forceinline__ void heads_block(const HeadArgs& a, const BlockPair b, const uint8_t* in, uint8_t* out,
                                            const uint32_t* in_sc, uint32_t* out_sc) {
  const uint8_t* sb = in + int64_t(b.src) * a.s_blk + slot_src(b.slots) * a.s_slot;
  uint8_t* db = out + int64_t(b.dst) * a.d_blk + slot_dst(b.slots) * a.d_slot;
  // buffer resources over one block's bytes from the slice's first row on
  // (every offset below stays inside the block)
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(sb), (short)0, int(a.s_blk), kBufferWord3);
  const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(db, (short)0, int(a.d_blk), kBufferWord3);
  const int rows = a.nh * b.nslots;
  const int total = rows * a.vpr;
  for (int base = 0; base < total; base += kHeadThreads * kHeadUnroll) {
    v4u r[kHeadUnroll];
    int doff[kHeadUnroll];
#pragma unroll
    for (int k = 0; k < kHeadUnroll; ++k) {
      const int i = base + k * kHeadThreads + int(threadIdx.x);
      if (i < total) {
        const int v = i % a.vpr;
        const int row = i / a.vpr;
        int h, s;
        if (a.dst_head_major) {
          h = row / b.nslots;
          s = row - h * b.nslots;
        } else {
          s = row / a.nh;
          h = row - s * a.nh;
        }
        r[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, int(s * a.s_slot + h * a.s_head) + v * 16, 0, KVX_LD_AUX);
        doff[k] = int(s * a.d_slot + h * a.d_head) + v * 16;
      }
    }
#pragma unroll
    for (int k = 0; k < kHeadUnroll; ++k) {
      const int i = base + k * kHeadThreads + int(threadIdx.x);
      if (i < total) __builtin_amdgcn_raw_buffer_store_b128(r[k], rd, doff[k], 0, KVX_HEAD_ST_AUX);
    }
  }
  if (out_sc && threadIdx.x == 0) out_sc[b.dst] = in_sc[b.src];
}

__global__ __launch_bounds__(kHeadThreads) void heads_kernel(HeadArgs a) {
  const int kv = blockIdx.y;
  heads_block(a, a.blocks[blockIdx.x], a.in[kv], a.out[kv], a.in_sc[kv], a.out_sc[kv]);
}

// Several layers of one plan's head transform in one launch
// (kvx_copy_heads_layers): workgroup x moves planned block x mod `per` of
// layer entry x / `per`, with the strides and the block list of `c`.
struct HeadLayer {
  const uint8_t* in[2];
  uint8_t* out[2];
  const uint32_t* in_sc[2];
  uint32_t* out_sc[2];
};
constexpr int kHeadLayersMax = 32;
struct HeadManyArgs {
  HeadArgs c;
  int32_t n, per;  // layer entries; planned blocks per entry
  HeadLayer e[kHeadLayersMax];
};

__global__ __launch_bounds__(kHeadThreads) void heads_many_kernel(HeadManyArgs a) {
  const int kv = blockIdx.y;
  const int lo = int(blockIdx.x) / a.per;
  const int bi = int(blockIdx.x) - lo * a.per;
  const HeadLayer& e = a.e[lo];
  heads_block(a.c, a.c.blocks[bi], e.in[kv], e.out[kv], e.in_sc[kv], e.out_sc[kv]);
}

// One shared piece list: one y row per region; one list per region: the tags.
static unsigned grid_y(const kvx_plan_t* p) { return p->nlists == 1 ? unsigned(p->nreg) : 1u; }

// Enqueue the copy kernel of shape (T, V) for one layer; `in`/`out` and the
// scale pointers are already resolved for the mode.  Splits very long work
// lists.
template <int MODE, int T, int V>
static int launch_copy_shape(kvx_plan_t* p, CopyArgs a, int64_t scale_slots, hipStream_t s, hipEvent_t started,
                             hipEvent_t finished, int64_t* launches) {
  const int64_t np = int64_t(p->pieces.size());
  const bool scales = a.in_sc[0] != nullptr;
  const unsigned gy = grid_y(p);
  const int64_t nsw = scales ? (scale_slots + T - 1) / T : 0;
  a.blocks = p->d_blocks;
  a.n_blocks = int32_t(p->blocks.size());
  a.n_scale_slots = int32_t(scale_slots);
  int64_t first = 0;
  // Pieces in chunks of kMaxGridX; the scale workgroups ride on the last chunk.
  do {
    if (launches) ++*launches;
    const int64_t cnt = std::min<int64_t>(np - first, kMaxGridX);
    const bool last = first + cnt >= np;
    a.pieces = p->d_pieces + first;
    a.n_pieces = int32_t(cnt);
    const bool on = xcd_on(T * V == 256, cnt);
    a.xcd = on;
    a.first_scale_wg = int32_t(xcd_span(cnt, on));
    const int64_t gx = a.first_scale_wg + (last ? nsw : 0);
    if (gx > 0) {
      if (started || finished) {
        // timestamps come from the dispatch packet itself: no extra packets
        hipExtLaunchKernelGGL(copy_kernel<MODE, T, V>, dim3(unsigned(gx), gy), dim3(T), 0, s,
                              first == 0 ? started : nullptr, last ? finished : nullptr, 0u, a);
      } else {
        hipLaunchKernelGGL((copy_kernel<MODE, T, V>), dim3(unsigned(gx), gy), dim3(T), 0, s, a);
      }
    }
    first += cnt;
  } while (first < np);
  return check_launch("kvx copy kernel launch");
}

// Enqueue the run-table kernel for one layer (a run-mode plan).
template <int MODE>
static int launch_runs(kvx_plan_t* p, const CopyArgs& c, int64_t scale_slots, hipStream_t s, hipEvent_t started,
                       hipEvent_t finished, int64_t* launches) {
  RunArgs a{};
  a.runs = MODE == kPush ? p->d_runs_dst : p->d_runs_plan;
  a.gidx = MODE == kPush ? p->d_gidx_dst : p->d_gidx_plan;
  a.blocks = p->d_blocks;
  a.nruns = uint32_t(p->runs_dst.size());
  a.total16 = p->run_total16;
  a.n_chunks = int32_t((int64_t(p->run_total16) + kRunChunk16 - 1) / kRunChunk16);
  a.xcd = xcd_on(true, a.n_chunks);
  a.chunk_span = int32_t(xcd_span(a.n_chunks, a.xcd));
  a.n_blocks = int32_t(p->blocks.size());
  a.n_scale_slots = int32_t(scale_slots);
  const uint32_t src_region = uint32_t(int64_t(p->src.NB) * p->src.block_bytes());
  const uint32_t dst_region = uint32_t(int64_t(p->dst.NB) * p->dst.block_bytes());
  const uint32_t payload = uint32_t(int64_t(p->run_total16) * 16);
  a.in_bytes = MODE == kUnpack ? payload : src_region;
  a.out_bytes = MODE == kPack ? payload : dst_region;
  for (int r = 0; r < 2; ++r) {
    a.in[r] = c.in[r];
    a.out[r] = c.out[r];
    a.in_sc[r] = c.in_sc[r];
    a.out_sc[r] = c.out_sc[r];
  }
  const int64_t nsw = c.in_sc[0] ? (scale_slots + 255) / 256 : 0;
  const int64_t gx = (a.n_chunks ? a.chunk_span : 0) + nsw;
  if (gx == 0) return KVX_OK;
  if (gx > kMaxGridX) return fail(KVX_E_UNSUPPORTED, "kvx run-table launch: %lld workgroups", (long long)gx);
  hipExtLaunchKernelGGL(run_kernel<MODE>, dim3(unsigned(gx), grid_y(p)), dim3(256), 0, s, started, finished, 0u, a);
  if (launches) ++*launches;
  return check_launch("kvx run-table kernel launch");
}

template <int MODE>
static int launch_copy(kvx_plan_t* p, CopyArgs a, int64_t scale_slots, hipStream_t s,
                       hipEvent_t started = nullptr, hipEvent_t finished = nullptr, int64_t* launches = nullptr) {
  if (p->runs_mode) return launch_runs<MODE>(p, a, scale_slots, s, started, finished, launches);
  switch (p->shape) {
    case kShapeLong:
      return launch_copy_shape<MODE, kShapes[kShapeLong].threads, kShapes[kShapeLong].vecs>(
          p, a, scale_slots, s, started, finished, launches);
    case kShapeLongSmall:
      return launch_copy_shape<MODE, kShapes[kShapeLongSmall].threads, kShapes[kShapeLongSmall].vecs>(
          p, a, scale_slots, s, started, finished, launches);
    default:
      return launch_copy_shape<MODE, kShapes[kShapeFine].threads, kShapes[kShapeFine].vecs>(
          p, a, scale_slots, s, started, finished, launches);
  }
}

// `started` / `finished` (nullable): timestamps of this launch's dispatch
// (hipExtLaunchKernelGGL adds no queue packets for them).
template <int MODE>
static void launch_many(const ManyArgs& m, int32_t shape, unsigned gy, hipStream_t s,
                        hipEvent_t started, hipEvent_t finished) {
  const dim3 grid(unsigned(m.span), gy);
  switch (shape) {
    case kShapeLong:
      hipExtLaunchKernelGGL((copy_many_kernel<MODE, kShapes[kShapeLong].threads, kShapes[kShapeLong].vecs>), grid,
                            dim3(kShapes[kShapeLong].threads), 0, s, started, finished, 0u, m);
      break;
    case kShapeLongSmall:
      hipExtLaunchKernelGGL(
          (copy_many_kernel<MODE, kShapes[kShapeLongSmall].threads, kShapes[kShapeLongSmall].vecs>), grid,
          dim3(kShapes[kShapeLongSmall].threads), 0, s, started, finished, 0u, m);
      break;
    default:
      hipExtLaunchKernelGGL((copy_many_kernel<MODE, kShapes[kShapeFine].threads, kShapes[kShapeFine].vecs>), grid,
                            dim3(kShapes[kShapeFine].threads), 0, s, started, finished, 0u, m);
  }
}

// Entries of one mode batched into as few launches as the limits allow:
// entries with the same grid height share a launch, in their order (up to
// kManyMax entries and kMaxGridX workgroups), and the entries' scale copies,
// if any, follow in one small launch behind it.  A launch whose entries all
// take the same one-wave shape and together stay within one round of it (at
// most kLongMaxPieces pieces of 32 KiB) runs in that shape; any other launch
// streams its pieces as 4 KiB chunks of four-wave workgroups, the shape that
// copies long launches fastest, taking each plan's pieces in destination
// order.
template <int MODE>
class ManyBatch {
 public:
  // With `started` / `finished`, the first launch records its start into
  // `started` and every launch its end into `finished` (the last one wins).
  explicit ManyBatch(hipStream_t s, hipEvent_t started = nullptr, hipEvent_t finished = nullptr)
      : s_(s), started_(started), finished_(finished) {}

  // Whether plan p's pieces fit a batched launch at all.
  // (Run-table plans have no pieces: they launch alone.)
  static bool fits(const kvx_plan_t* p) {
    return !p->runs_mode && (int64_t(p->pieces.size()) << piece_shift(p->shape)) <= kMaxGridX;
  }

  // Entries of one-region and of two-region plans gather in launches of
  // their own (the grid height is the region count), each in arrival order,
  // so that interleaved layer groups of a hybrid model (attention layers
  // beside state or latent layers) still fill whole launches.
  // The copy of `a` (region bases, and scale pointers when the pools hold
  // scales) over plan p's pieces; `scale_slots` scale entries per region.
  int add(const kvx_plan_t* p, const CopyArgs& a, int64_t scale_slots) {
    const int64_t np = int64_t(p->pieces.size());
    if (np == 0) return KVX_OK;
    const int32_t shift = piece_shift(p->shape);
    Group& g = g_[grid_y(p) - 1];
    if (g.m.n == kManyMax || (g.m.n > 0 && g.fine + (np << shift) > kMaxGridX)) {
      const int rc = flush_group(g);
      if (rc) return rc;
    }
    if (g.m.n == 0) g.seq = ++seq_;
    g.shape = g.m.n == 0 || p->shape == g.shape ? p->shape : -1;
    g.gy = grid_y(p);
    ManyEntry& e = g.m.e[g.m.n];
    e.pieces = p->d_pieces;
    g.stream[g.m.n] = p->d_stream;
    for (int r = 0; r < 2; ++r) {
      e.in[r] = r < p->nreg ? a.in[r] : nullptr;
      e.out[r] = r < p->nreg ? a.out[r] : nullptr;
    }
    g.np[g.m.n] = int32_t(np);
    g.shift[g.m.n] = shift;
    ++g.m.n;
    g.n32 += p->n32;
    g.fine += np << shift;
    if (a.in_sc[0] && scale_slots > 0) {
      ScaleEntry& se = g.sm.e[g.sm.n++];
      se.blocks = p->d_blocks;
      for (int r = 0; r < 2; ++r) {
        se.in_sc[r] = r < p->nreg ? a.in_sc[r] : nullptr;
        se.out_sc[r] = r < p->nreg ? a.out_sc[r] : nullptr;
      }
      se.n_blocks = int32_t(p->blocks.size());
      se.n_slots = int32_t(scale_slots);
      se.first = int32_t(g.swg);
      g.swg += (scale_slots + kScaleThreads - 1) / kScaleThreads;
    }
    return KVX_OK;
  }

  // Launch whatever is gathered, the group started first first.
  int flush() {
    Group* a = &g_[0];
    Group* b = &g_[1];
    if (b->m.n && (!a->m.n || b->seq < a->seq)) std::swap(a, b);
    int rc = flush_group(*a);
    if (!rc) rc = flush_group(*b);
    return rc;
  }

  // A launch outside the batch (a pair with scales) takes over the start
  // timestamp when it comes first.
  hipEvent_t take_started() {
    hipEvent_t e = started_;
    started_ = nullptr;
    return e;
  }
  hipEvent_t finished() const { return finished_; }
  // Kernel launches enqueued by flush so far.
  int64_t launches() const { return launches_; }

 private:
  struct Group {
    ManyArgs m{};
    int64_t n32 = 0;   // 32 KiB pieces in the launch (all regions)
    int64_t fine = 0;  // workgroups of the launch in the 4 KiB shape
    unsigned gy = 0;
    int32_t shape = -1;  // common shape of the entries, -1 when they differ
    int64_t seq = 0;     // order of the group's first entry
    ScaleManyArgs sm{};  // the entries' scale copies (entries with scales only)
    int64_t swg = 0;     // their workgroups
    int32_t np[kManyMax] = {};
    int32_t shift[kManyMax] = {};
    const Piece* stream[kManyMax] = {};  // each entry's pieces in streaming order
  };

  int flush_group(Group& g) {
    if (g.m.n == 0) return KVX_OK;
    const bool keep = (g.shape == kShapeLong || g.shape == kShapeLongSmall) && g.n32 <= kLongMaxPieces;
    int64_t total = 0;
    for (int32_t j = 0; j < g.m.n; ++j) {
      g.m.e[j].first = int32_t(total);
      g.m.e[j].shift = keep ? 0 : g.shift[j];
      if (!keep) g.m.e[j].pieces = g.stream[j];
      total += int64_t(g.np[j]) << g.m.e[j].shift;
    }
    g.m.items = int32_t(total);
    g.m.uniform = total % g.m.n == 0 ? int32_t(total / g.m.n) : 0;
    for (int32_t j = 0; j < g.m.n; ++j)
      if (g.m.e[j].first != j * g.m.uniform) g.m.uniform = 0;  // then x / uniform < n for every x < items
    g.m.xcd = xcd_on(!keep, total);
    g.m.span = int32_t(xcd_span(total, g.m.xcd));
    launch_many<MODE>(g.m, keep ? g.shape : int32_t(kShapeFine), g.gy, s_, started_, finished_);
    started_ = nullptr;
    ++launches_;
    if (g.sm.n > 0) {  // the scales: a small launch of their own behind the payload's
      hipExtLaunchKernelGGL(scale_many_kernel<MODE>, dim3(unsigned(g.swg), g.gy), dim3(kScaleThreads), 0, s_,
                            nullptr, finished_, 0u, g.sm);
      ++launches_;
    }
    g.m.n = 0;
    g.sm.n = 0;
    g.swg = 0;
    g.n32 = 0;
    g.fine = 0;
    g.shape = -1;
    return check_launch("kvx copy_many kernel launch");
  }

  hipStream_t s_;
  hipEvent_t started_, finished_;
  int64_t launches_ = 0;
  int64_t seq_ = 0;
  Group g_[2];
};

// ---------------------------------------------------------------------------
// Work lists without allocation (kvx_plan_noalloc): one static scratch array
// per device holds the work list of the most recent plan built that way.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

struct ScratchSlot {
  std::atomic<char*> ptr{nullptr};     // the device address of `scratch` on this device
  std::atomic<uint64_t> gen{0};        // bumped by every kvx_plan_noalloc on this device
};
static ScratchSlot g_scratch[kMaxDevices];
static std::mutex g_scratch_mu;

// The device address of the scratch array on the current device, looked up
// once per device (the host-side name is not a device address).
static int scratch_ptr(int device, char** out) {
  if (device < 0 || device >= kMaxDevices) return fail(KVX_E_UNSUPPORTED, "kvx_plan_noalloc: device %d", device);
  ScratchSlot& sl = g_scratch[device];
  char* p = sl.ptr.load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    p = sl.ptr.load(std::memory_order_relaxed);
    if (!p) {
      void* addr = nullptr;
      const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return fail_hip(e, "kvx_plan_noalloc: hipGetSymbolAddress(scratch)");
      p = static_cast<char*>(addr);
      sl.ptr.store(p, std::memory_order_release);
    }
  }
  *out = p;
  return KVX_OK;
}

static int check_device_plan(const kvx_plan_t* p, const char* fn) {
  if (!p) return fail(KVX_E_INVAL, "%s: null plan", fn);
  if (p->host_only) return fail(KVX_E_INVAL, "%s: plan was built host-only", fn);
  if (p->in_scratch && g_scratch[p->device].gen.load(std::memory_order_acquire) != p->scratch_gen)
    return fail(KVX_E_INVAL, "%s: the plan's work list in the device scratch array was replaced by a later "
                "kvx_plan_noalloc", fn);
  return KVX_OK;
}

static CopyArgs push_args(const kvx_plan_t* p, int32_t layer) {
  CopyArgs a{};
  for (int r = 0; r < p->nreg; ++r) {
    a.in[r] = static_cast<const uint8_t*>(p->src.base(r, layer));
    a.out[r] = static_cast<uint8_t*>(p->dst.base(r, layer));
    if (p->src.scales) {
      a.in_sc[r] = reinterpret_cast<const uint32_t*>(p->src.scale(r, layer));
      a.out_sc[r] = reinterpret_cast<uint32_t*>(p->dst.scale(r, layer));
    }
  }
  return a;
}

int check_push_pair(const kvx_plan_t* p, int32_t layer, const char* fn, int32_t i) {
  int rc = check_device_plan(p, fn);
  if (rc) return rc;
  if (!p->push_ok) return fail(KVX_E_MISMATCH, "%s: pair %d: pools differ in head count or layout", fn, i);
  if (layer < 0 || layer >= p->src.L)
    return fail(KVX_E_RANGE, "%s: pair %d: layer %d outside [0,%d)", fn, i, layer, p->src.L);
  return KVX_OK;
}

int push_batch(const kvx_plan_t* const* plans, const int32_t* layers, int32_t n, hipStream_t stream,
               hipEvent_t started, hipEvent_t finished, int64_t* launches) {
  int64_t alone = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int rc = enqueue_waits(const_cast<kvx_plan_t*>(plans[i]), nullptr, stream);
    if (rc) return rc;
  }
  // Pairs share launches (ManyBatch; their scales, if any, a small launch
  // behind the payload's); a pair with too many pieces for one launch, or a
  // run-table plan, is launched alone, in order.
  ManyBatch<kPush> batch(stream, started, finished);
  for (int32_t i = 0; i < n; ++i) {
    kvx_plan_t* p = const_cast<kvx_plan_t*>(plans[i]);
    int rc;
    if (!ManyBatch<kPush>::fits(p)) {
      if (p->pieces.empty() && p->blocks.empty()) continue;
      rc = batch.flush();
      if (rc) return rc;
      rc = launch_copy<kPush>(p, push_args(p, layers[i]), int64_t(p->blocks.size()), stream,
                              batch.take_started(), batch.finished(), &alone);
      if (rc) return rc;
      continue;
    }
    rc = batch.add(p, push_args(p, layers[i]), int64_t(p->blocks.size()));
    if (rc) return rc;
  }
  const int rc = batch.flush();
  if (launches) *launches += alone + batch.launches();
  return rc;
}

}  // namespace kvx

using namespace kvx;

extern "C" {

int kvx_push_layer(const kvx_plan_t* cp, int32_t layer, hipEvent_t ready, hipStream_t stream) {
  return kvx_push_layer_timed(cp, layer, ready, stream, nullptr, nullptr);
}

int kvx_push_layer_timed(const kvx_plan_t* cp, int32_t layer, hipEvent_t ready, hipStream_t stream,
                         hipEvent_t started, hipEvent_t finished) {
  int rc = check_device_plan(cp, "kvx_push_layer");
  if (rc) return rc;
  kvx_plan_t* p = const_cast<kvx_plan_t*>(cp);
  if (!p->push_ok) return fail(KVX_E_MISMATCH, "kvx_push_layer: pools differ in head count or layout");
  if (layer < 0 || layer >= p->src.L)
    return fail(KVX_E_RANGE, "kvx_push_layer: layer %d outside [0,%d)", layer, p->src.L);
  rc = enqueue_waits(p, ready, stream);
  if (rc) return rc;
  if (p->pieces.empty() && p->blocks.empty()) return KVX_OK;
  return launch_copy<kPush>(p, push_args(p, layer), int64_t(p->blocks.size()), stream, started, finished);
}

int kvx_push_many(const kvx_plan_t* const* plans, const int32_t* layers, int32_t n, hipEvent_t ready,
                  hipStream_t stream) {
  return kvx_push_many_timed(plans, layers, n, ready, stream, nullptr, nullptr);
}

int kvx_push_many_timed(const kvx_plan_t* const* plans, const int32_t* layers, int32_t n, hipEvent_t ready,
                        hipStream_t stream, hipEvent_t started, hipEvent_t finished) {
  if (n < 0 || (n > 0 && (!plans || !layers))) return fail(KVX_E_INVAL, "kvx_push_many: bad arguments");
  for (int32_t i = 0; i < n; ++i) {
    int rc = check_push_pair(plans[i], layers[i], "kvx_push_many", i);
    if (rc) return rc;
  }
  int rc = wait_event(ready, stream);
  if (rc) return rc;
  return kvx::push_batch(plans, layers, n, stream, started, finished);
}

static int staging_call(const kvx_plan_t* cp, int32_t l0, int32_t l1, const void* staging,
                        int64_t cap, const char* fn, kvx_plan_t** out) {
  int rc = check_device_plan(cp, fn);
  if (rc) return rc;
  kvx_plan_t* p = const_cast<kvx_plan_t*>(cp);
  if (!p->push_ok) return fail(KVX_E_MISMATCH, "%s: pools differ in head count or layout", fn);
  if (l0 < 0 || l1 < l0 || l1 > p->src.L)
    return fail(KVX_E_RANGE, "%s: layers [%d,%d) outside [0,%d]", fn, l0, l1, p->src.L);
  const int64_t need = int64_t(l1 - l0) * p->stg_layer();
  if (need > 0 && !staging) return fail(KVX_E_INVAL, "%s: null staging buffer", fn);
  if (cap < need) return fail(KVX_E_INVAL, "%s: staging holds %lld bytes, needs %lld", fn,
                              (long long)cap, (long long)need);
  if (uintptr_t(staging) & 15) return fail(KVX_E_UNSUPPORTED, "%s: staging not 16-byte aligned", fn);
  *out = p;
  return KVX_OK;
}

int kvx_pack(const kvx_plan_t* cp, int32_t l0, int32_t l1, void* staging, int64_t cap,
             hipStream_t stream) {
  kvx_plan_t* p = nullptr;
  int rc = staging_call(cp, l0, l1, staging, cap, "kvx_pack", &p);
  if (rc) return rc;
  rc = enqueue_waits(p, nullptr, stream);
  if (rc) return rc;
  const int64_t layer_bytes = p->stg_layer();
  if (layer_bytes == 0) return KVX_OK;
  uint8_t* stg = static_cast<uint8_t*>(staging);
  const bool many = ManyBatch<kPack>::fits(p);  // several layers per launch
  ManyBatch<kPack> batch(stream);
  for (int32_t l = l0; l < l1; ++l) {
    CopyArgs a{};
    for (int r = 0; r < p->nreg; ++r) {
      uint8_t* reg = stg + int64_t(l - l0) * layer_bytes + p->stg_offset(r);
      a.in[r] = static_cast<const uint8_t*>(p->src.base(r, l));
      a.out[r] = reg;
      if (p->src.scales) {
        a.in_sc[r] = reinterpret_cast<const uint32_t*>(p->src.scale(r, l));
        a.out_sc[r] = reinterpret_cast<uint32_t*>(reg + p->payload[r]);
      }
    }
    rc = many ? batch.add(p, a, p->scale_seg_bytes / 4) : launch_copy<kPack>(p, a, p->scale_seg_bytes / 4, stream);
    if (rc) return rc;
  }
  return batch.flush();
}

int kvx_unpack(const kvx_plan_t* cp, int32_t l0, int32_t l1, const void* staging, int64_t cap,
               hipStream_t stream) {
  kvx_plan_t* p = nullptr;
  int rc = staging_call(cp, l0, l1, staging, cap, "kvx_unpack", &p);
  if (rc) return rc;
  rc = enqueue_waits(p, nullptr, stream);
  if (rc) return rc;
  const int64_t layer_bytes = p->stg_layer();
  if (layer_bytes == 0) return KVX_OK;
  const uint8_t* stg = static_cast<const uint8_t*>(staging);
  const bool many = ManyBatch<kUnpack>::fits(p);  // several layers per launch
  ManyBatch<kUnpack> batch(stream);
  for (int32_t l = l0; l < l1; ++l) {
    CopyArgs a{};
    for (int r = 0; r < p->nreg; ++r) {
      const uint8_t* reg = stg + int64_t(l - l0) * layer_bytes + p->stg_offset(r);
      a.in[r] = reg;
      a.out[r] = static_cast<uint8_t*>(p->dst.base(r, l));
      if (p->dst.scales) {
        a.in_sc[r] = reinterpret_cast<const uint32_t*>(reg + p->payload[r]);
        a.out_sc[r] = reinterpret_cast<uint32_t*>(p->dst.scale(r, l));
      }
    }
    const int64_t slots = int64_t(p->blocks.size());
    rc = many ? batch.add(p, a, slots) : launch_copy<kUnpack>(p, a, slots, stream);
    if (rc) return rc;
  }
  return batch.flush();
}

int kvx_plan_noalloc(const kvx_pool* src, const kvx_pool* dst, int32_t num_requests, const int64_t* num_tokens,
                     const int64_t* src_offsets, const int64_t* dst_offsets, const int32_t* src_ids,
                     const int32_t* dst_ids, uint32_t flags, hipStream_t upload_stream, kvx_plan_t** out) {
  if (!out) return fail(KVX_E_INVAL, "kvx_plan_noalloc: null output");
  if (flags & KVX_PLAN_HOST_ONLY) return fail(KVX_E_INVAL, "kvx_plan_noalloc: a host-only plan has no work list");
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return fail_hip(e, "kvx_plan_noalloc: hipGetDevice");
  char* buf = nullptr;
  int rc = scratch_ptr(device, &buf);
  if (rc) return rc;
  kvx_plan_t* p = nullptr;
  rc = plan_build(src, dst, num_requests, num_tokens, src_offsets, dst_offsets, src_ids, dst_ids, flags,
                  upload_stream, &p);
  if (rc) return rc;
  const size_t need = worklist_bytes(p);
  if (need > kScratchBytes) {
    plan_free_idle(p);
    return fail(KVX_E_NOMEM, "kvx_plan_noalloc: the work list needs %zu bytes, the scratch array holds %zu "
                "(build with kvx_plan, or with KVX_PLAN_RUNS for a smaller streaming work list)",
                need, kScratchBytes);
  }
  p->device = device;
  p->in_scratch = true;
  p->scratch_gen = g_scratch[device].gen.fetch_add(1, std::memory_order_acq_rel) + 1;
  p->dev_buf = buf;
  p->dev_bytes = need;
  rc = worklist_copy(p, buf, upload_stream);
  if (rc == KVX_OK) {
    // no event: the upload is waited for here, so device calls need no wait
    e = hipStreamSynchronize(upload_stream);
    if (e != hipSuccess) rc = fail_hip(e, "kvx_plan_noalloc: hipStreamSynchronize(upload)");
  }
  if (rc) {
    plan_free_idle(p);
    return rc;
  }
  p->upload_seen.store(true, std::memory_order_release);
  *out = p;
  return KVX_OK;
}

}  // extern "C"

// Checks shared by the head-transform calls, for layers [l0, l1).
static int heads_check(const kvx_plan_t* cp, int64_t l0, int64_t l1, int32_t src_head0, int32_t dst_head0,
                       int32_t num_heads, const char* fn) {
  int rc = check_device_plan(cp, fn);
  if (rc) return rc;
  if (cp->src.state) return fail(KVX_E_MISMATCH, "%s: state pools have no heads", fn);
  if (src_head0 < 0 || dst_head0 < 0 || num_heads < 0)
    return fail(KVX_E_INVAL, "%s: negative head index or count", fn);
  if (l0 < 0 || l1 < l0 || l1 > cp->src.L)
    return fail(KVX_E_RANGE, "%s: layers [%lld,%lld) outside [0,%d)", fn, (long long)l0, (long long)l1, cp->src.L);
  if (int64_t(src_head0) + num_heads > cp->src.H || int64_t(dst_head0) + num_heads > cp->dst.H)
    return fail(KVX_E_RANGE, "%s: head slice [%d,+%d) -> [%d,+%d) outside %d / %d heads", fn, src_head0,
                num_heads, dst_head0, num_heads, cp->src.H, cp->dst.H);
  return KVX_OK;
}

// Strides and slice of a plan's head transform (no layer bases yet).
static HeadArgs heads_common(const kvx_plan_t* p, int32_t num_heads) {
  const Geom& gs = p->src;
  const Geom& gd = p->dst;
  HeadArgs a{};
  a.s_blk = gs.block_bytes();
  a.s_slot = gs.slot_stride();
  a.s_head = gs.head_stride();
  a.d_blk = gd.block_bytes();
  a.d_slot = gd.slot_stride();
  a.d_head = gd.head_stride();
  a.vpr = int32_t(gs.row_bytes() / 16);
  a.nh = num_heads;
  a.dst_head_major = gd.layout == KVX_HND;
  return a;
}

// Region bases of one layer's head slice.
static HeadLayer heads_layer(const kvx_plan_t* p, int32_t layer, int32_t src_head0, int32_t dst_head0) {
  const Geom& gs = p->src;
  const Geom& gd = p->dst;
  HeadLayer e{};
  for (int r = 0; r < p->nreg; ++r) {
    e.in[r] = static_cast<const uint8_t*>(gs.base(r, layer)) + int64_t(src_head0) * gs.head_stride();
    e.out[r] = static_cast<uint8_t*>(gd.base(r, layer)) + int64_t(dst_head0) * gd.head_stride();
    if (gs.scales) {
      e.in_sc[r] = reinterpret_cast<const uint32_t*>(gs.scale(r, layer));
      e.out_sc[r] = reinterpret_cast<uint32_t*>(gd.scale(r, layer));
    }
  }
  return e;
}

// One layer, in launches of at most kMaxGridX planned blocks, each
// recording its end into `finished` (nullable).
static int64_t heads_launch_layer(const kvx_plan_t* p, const HeadArgs& common, const HeadLayer& e, hipStream_t stream,
                                  hipEvent_t finished = nullptr) {
  HeadArgs a = common;
  for (int r = 0; r < 2; ++r) {
    a.in[r] = e.in[r];
    a.out[r] = e.out[r];
    a.in_sc[r] = e.in_sc[r];
    a.out_sc[r] = e.out_sc[r];
  }
  const int64_t nb = int64_t(p->blocks.size());
  int64_t launches = 0;
  for (int64_t first = 0; first < nb; first += kMaxGridX) {
    const int64_t cnt = std::min<int64_t>(nb - first, kMaxGridX);
    a.blocks = p->d_blocks + first;
    hipExtLaunchKernelGGL(heads_kernel, dim3(unsigned(cnt), unsigned(p->nreg)), dim3(kHeadThreads), 0, stream,
                          nullptr, finished, 0u, a);
    ++launches;
  }
  return launches;
}

// Launches of up to kHeadLayersMax layers of one plan and head slice
// (kvx_copy_heads_layers and the write queue), one per layer when a layer's
// planned blocks alone fill half a launch; every launch records its end into
// `finished` (nullable).  Returns the launches enqueued.
static int64_t heads_launch_layers(const kvx_plan_t* p, const int32_t* layers, int32_t n, int32_t src_head0,
                                   int32_t dst_head0, int32_t num_heads, hipStream_t stream, hipEvent_t finished) {
  if (p->blocks.empty() || num_heads == 0 || n == 0) return 0;
  const HeadArgs common = heads_common(p, num_heads);
  const int64_t nb = int64_t(p->blocks.size());
  int64_t launches = 0;
  if (nb > kMaxGridX / 2) {
    for (int32_t j = 0; j < n; ++j)
      launches += heads_launch_layer(p, common, heads_layer(p, layers[j], src_head0, dst_head0), stream, finished);
    return launches;
  }
  const int32_t per_launch = int32_t(std::min<int64_t>(kHeadLayersMax, kMaxGridX / nb));
  HeadManyArgs m{};
  m.c = common;
  m.c.blocks = p->d_blocks;
  m.per = int32_t(nb);
  for (int32_t j0 = 0; j0 < n; j0 += per_launch) {
    m.n = std::min(per_launch, n - j0);
    for (int32_t j = 0; j < m.n; ++j) m.e[j] = heads_layer(p, layers[j0 + j], src_head0, dst_head0);
    hipExtLaunchKernelGGL(heads_many_kernel, dim3(unsigned(int64_t(m.n) * nb), unsigned(p->nreg)),
                          dim3(kHeadThreads), 0, stream, nullptr, finished, 0u, m);
    ++launches;
  }
  return launches;
}

int kvx::check_heads_write(const HeadsWrite& w, const char* fn) {
  return heads_check(w.plan, w.layer, int64_t(w.layer) + 1, w.src_head0, w.dst_head0, w.num_heads, fn);
}

int kvx::heads_batch(const HeadsWrite* w, int32_t n, hipStream_t stream, hipEvent_t finished, int64_t* launches) {
  for (int32_t i = 0; i < n; ++i) {
    const int rc = enqueue_waits(const_cast<kvx_plan_t*>(w[i].plan), nullptr, stream);
    if (rc) return rc;
  }
  std::vector<int32_t> layers;
  int64_t count = 0;
  for (int32_t i = 0; i < n;) {
    int32_t j = i;
    layers.clear();
    while (j < n && w[j].plan == w[i].plan && w[j].src_head0 == w[i].src_head0 &&
           w[j].dst_head0 == w[i].dst_head0 && w[j].num_heads == w[i].num_heads)
      layers.push_back(w[j++].layer);
    count += heads_launch_layers(w[i].plan, layers.data(), int32_t(layers.size()), w[i].src_head0, w[i].dst_head0,
                                 w[i].num_heads, stream, finished);
    i = j;
  }
  if (launches) *launches += count;
  return count ? check_launch("kvx heads kernel launch") : KVX_OK;
}

extern "C" {

int kvx_copy_heads(const kvx_plan_t* cp, int32_t layer, int32_t src_head0, int32_t dst_head0,
                   int32_t num_heads, hipEvent_t ready, hipStream_t stream) {
  int rc = heads_check(cp, layer, int64_t(layer) + 1, src_head0, dst_head0, num_heads, "kvx_copy_heads");
  if (rc) return rc;
  kvx_plan_t* p = const_cast<kvx_plan_t*>(cp);
  rc = enqueue_waits(p, ready, stream);
  if (rc) return rc;
  if (p->blocks.empty() || num_heads == 0) return KVX_OK;
  heads_launch_layer(p, heads_common(p, num_heads), heads_layer(p, layer, src_head0, dst_head0), stream);
  return check_launch("kvx heads kernel launch");
}

int kvx_copy_heads_layers(const kvx_plan_t* cp, int32_t l0, int32_t l1, int32_t src_head0, int32_t dst_head0,
                          int32_t num_heads, hipEvent_t ready, hipStream_t stream) {
  int rc = heads_check(cp, l0, l1, src_head0, dst_head0, num_heads, "kvx_copy_heads_layers");
  if (rc) return rc;
  kvx_plan_t* p = const_cast<kvx_plan_t*>(cp);
  rc = enqueue_waits(p, ready, stream);
  if (rc) return rc;
  if (p->blocks.empty() || num_heads == 0 || l1 == l0) return KVX_OK;
  std::vector<int32_t> layers;
  for (int32_t l = l0; l < l1; ++l) layers.push_back(l);
  heads_launch_layers(p, layers.data(), l1 - l0, src_head0, dst_head0, num_heads, stream, nullptr);
  return check_launch("kvx heads kernel launch");
}

}  // extern "C"
