// Internal types shared by the libkvx host code (kvx_host.cpp) and the HIP
// kernels (kvx_kernels.hip).  Not part of the ABI.
#pragma once

#include <atomic>
#include <cstdint>
#include <string>
#include <vector>

#include "kvx.h"

namespace kvx {

// One workgroup's share of a (layer, region) pair: a contiguous byte range
// on the source side, on the destination side and inside the staging region.
// All offsets are region-relative and identical for every layer, so one list
// serves every launch.  When all regions share one triple list (K and V) the
// launch's y index picks the region and `reg` is 0; when each region has its
// own list (state slots) the pieces of all lists are concatenated and `reg`
// names the region.  32 bytes: read with one scalar load per workgroup.
struct Piece {
  int64_t src_off;
  int64_t dst_off;
  int64_t stg_off;
  int32_t len;  // bytes, multiple of 16, <= the plan's piece size
  int32_t reg;  // region offset added to blockIdx.y
};
static_assert(sizeof(Piece) == 32, "Piece is 32 bytes");

// One planned block: (source block, destination block, tokens it holds).
// With different block sizes per side it is a piece of a token range that
// stays inside one source and one destination block, starting at slot
// `slots & 0xffff` of the source block and `slots >> 16` of the destination
// block (both 0 with equal block sizes).
struct BlockPair {
  int32_t src, dst, nslots, slots;
};
static_assert(sizeof(BlockPair) == 16, "BlockPair is 16 bytes");
inline int32_t pack_slots(int64_t src_slot, int64_t dst_slot) { return int32_t(src_slot | (dst_slot << 16)); }
__host__ __device__ inline int32_t slot_src(int32_t slots) { return slots & 0xffff; }
__host__ __device__ inline int32_t slot_dst(int32_t slots) { return (slots >> 16) & 0xffff; }

// Launch shapes of the layer copy kernels: lanes per workgroup and 16-byte
// vectors each lane keeps in flight; a workgroup copies one piece of at most
// lanes x vectors x 16 bytes.  A plan picks one shape for all its pieces
// from its own triples (pick_shape in kvx_host.cpp).
enum CopyShape : int32_t {
  kShapeLong = 0,       // one wave64 x 32 vectors: 32 KiB pieces
  kShapeLongSmall = 1,  // one wave64 x 16 vectors: 16 KiB pieces
  kShapeFine = 2,       // four wave64 x 1 vector: 4 KiB pieces
};
constexpr int kNumShapes = 3;
struct ShapeDims {
  int32_t threads, vecs;
};
constexpr ShapeDims kShapes[kNumShapes] = {{64, 32}, {64, 16}, {256, 1}};
constexpr int64_t shape_piece_bytes(int32_t s) { return int64_t(kShapes[s].threads) * kShapes[s].vecs * 16; }
// log2 of the 4 KiB chunks in one piece of shape s (kvx_push_many runs any
// plan's pieces as such chunks when its launch streams).
constexpr int32_t piece_shift(int32_t s) {
  return shape_piece_bytes(s) == 32768 ? 3 : shape_piece_bytes(s) == 16384 ? 2 : 0;
}
static_assert(shape_piece_bytes(kShapeFine) == 4096, "chunks of kvx_push_many are 4 KiB");
static_assert(piece_shift(kShapeLong) == 3 && piece_shift(kShapeLongSmall) == 2, "piece sizes");
// One-wave workgroups of 32 KiB pieces copy fastest when one launch holds
// kLongMinPieces..kLongMaxPieces of them (about one round per SIMD); see
// pick_shape in kvx_host.cpp.
constexpr int64_t kLongMinPieces = 608;
constexpr int64_t kLongMaxPieces = 1312;

// Run-table work list (KVX_PLAN_RUNS): one record per triple, a range
// contiguous on both sides, with its position in the list's flat byte space
// (the triples back to back in the table's order).  Every field is in
// 16-byte units, so each fits 32 bits for regions and staging below 64 GiB
// (the kernels address inside a region with 32-bit byte offsets, so run
// tables are used for regions below 4 GiB).  A workgroup copies one 4 KiB
// chunk of the flat space; a run index entry names the first run of each
// group of kRunGroupChunks chunks, from which each wave walks the records
// (scalar loads) to the runs of its 64 units.
struct RunRec {
  uint32_t src16, dst16, len16, start16;
};
static_assert(sizeof(RunRec) == 16, "RunRec is 16 bytes");
constexpr int32_t kRunGroupChunks = 8;
constexpr int32_t kRunChunk16 = 256;  // a 4 KiB chunk in 16-byte units

// One side's layer group.  Attention pools: nreg regions (K and V, or one
// latent region) of NB blocks.  State pools: two regions of NB slots of
// slot_bytes[r] bytes; BS, H, D, E and layout are unused.
struct Geom {
  int32_t L = 0, NB = 0, BS = 0, H = 0, D = 0, E = 0, layout = 0;
  int32_t nreg = 2;
  int32_t window = 0;          // sliding window in positions, 0 = full attention
  bool state = false;
  int64_t slot_bytes[2] = {0, 0};
  bool scales = false;
  std::vector<void*> k, v;     // region 0 and region 1 bases per layer (v empty with one region)
  std::vector<float*> ks, vs;

  void* base(int r, int l) const { return r == 0 ? k[size_t(l)] : v[size_t(l)]; }
  float* scale(int r, int l) const { return r == 0 ? ks[size_t(l)] : vs[size_t(l)]; }

  int64_t row_bytes() const { return int64_t(D) * E; }
  int64_t token_bytes() const { return int64_t(H) * row_bytes(); }
  int64_t block_bytes() const { return int64_t(BS) * token_bytes(); }
  // byte strides of (block, slot, head) inside a region
  int64_t slot_stride() const { return layout == KVX_NHD ? token_bytes() : row_bytes(); }
  int64_t head_stride() const { return layout == KVX_NHD ? row_bytes() : int64_t(BS) * row_bytes(); }
};

}  // namespace kvx

struct kvx_pool {
  kvx::Geom g;
};

struct kvx_plan_s {
  kvx::Geom src, dst;
  bool push_ok = false;   // same head count and layout: triples and pieces exist
  bool host_only = false;
  int32_t nreg = 2;       // regions per layer
  int32_t nlists = 1;     // 1: one triple list shared by every region; 2: one per region
  int32_t shape = kvx::kShapeLong;  // launch shape of the copy kernels (CopyShape)
  int64_t n32 = 0;                  // 32 KiB pieces covering one layer's triples (all regions)
  bool overlap = false;             // KVX_PLAN_OVERLAP: launches of this plan overlap each other
  // KVX_PLAN_RUNS honoured: streaming launches read run tables, no pieces.
  // runs_dst: the triples in destination order (push), start16 = their flat
  // position; runs_plan: plan order, start16 = the staging offset (pack,
  // unpack).  gidx_*: first run of each group of kRunGroupChunks chunks.
  bool want_runs = false;           // KVX_PLAN_RUNS was passed
  bool runs_mode = false;
  uint32_t run_total16 = 0;         // flat length of the (shared) list, 16-byte units
  std::vector<kvx::RunRec> runs_dst, runs_plan;
  std::vector<uint32_t> gidx_dst, gidx_plan;
  std::vector<kvx_run> runs;
  std::vector<kvx_triple> triples[2];
  std::vector<kvx::Piece> pieces;     // list 0's pieces, then list 1's
  // One-wave plans only: the same pieces, each list in destination order,
  // for launches that stream them as 4 KiB chunks (empty otherwise).
  std::vector<kvx::Piece> stream_pieces;
  std::vector<kvx::BlockPair> blocks;
  int64_t payload[2] = {0, 0};  // moved bytes per (layer, region)
  int64_t scale_seg_bytes = 0;  // per region inside staging (16-B padded), 0 without scales

  const std::vector<kvx_triple>& region_triples(int r) const { return triples[nlists == 1 ? 0 : r]; }
  // Bytes of one region (payload and scale segment) inside a layer's staging,
  // the offset of region r inside the layer, and one layer's staging bytes.
  int64_t stg_region(int r) const { return payload[r] + scale_seg_bytes; }
  int64_t stg_offset(int r) const { return r == 0 ? 0 : stg_region(0); }
  int64_t stg_layer() const { return nreg == 1 ? stg_region(0) : stg_region(0) + stg_region(1); }

  // device side
  void* dev_buf = nullptr;   // from the work-list arena (desc_alloc)
  size_t dev_bytes = 0;
  int device = 0;
  const kvx::Piece* d_pieces = nullptr;
  const kvx::Piece* d_stream = nullptr;  // pieces in streaming order (d_pieces for streaming plans)
  const kvx::BlockPair* d_blocks = nullptr;
  const kvx::RunRec* d_runs_dst = nullptr;
  const kvx::RunRec* d_runs_plan = nullptr;
  const uint32_t* d_gidx_dst = nullptr;
  const uint32_t* d_gidx_plan = nullptr;
  hipEvent_t upload_ev = nullptr;
  std::atomic<bool> upload_seen{false};
  // Work list in the device's static scratch array (kvx_plan_noalloc): it
  // stays valid while the device's scratch generation is still scratch_gen.
  bool in_scratch = false;
  uint64_t scratch_gen = 0;
};

namespace kvx {

// Thread-local error message; returns `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail_hip(hipError_t e, const char* what);

// Make `stream` wait for `ev` unless it has already fired (NULL: nothing).
int wait_event(hipEvent_t ev, hipStream_t stream);
// True while `stream` is capturing a graph.
bool stream_capturing(hipStream_t stream);
// Before a device call: enqueue the wait for `ready` and for the plan upload.
int enqueue_waits(kvx_plan_t* plan, hipEvent_t ready, hipStream_t stream);
// After a launch: turn a launch error into KVX_E_HIP.
int check_launch(const char* what);

// Device memory for plan work lists on the current device: `bytes` rounded
// up to 256, from chunks the library keeps mapped (hipFree would
// synchronize the whole device).  desc_free returns a range for reuse; the
// caller guarantees no enqueued work still reads it.
int desc_alloc(size_t bytes, void** out, int* device);
void desc_free(void* p, size_t bytes, int device);

// Free a plan whose enqueued work is known to have finished (no device
// drain, unlike kvx_plan_destroy).
void plan_free_idle(kvx_plan_t* plan);

// Validate the arguments of kvx_plan and build a plan's host tables, without
// its device work list.
int plan_build(const kvx_pool* src, const kvx_pool* dst, int32_t num_requests, const int64_t* num_tokens,
               const int64_t* src_offsets, const int64_t* dst_offsets, const int32_t* src_ids,
               const int32_t* dst_ids, uint32_t flags, hipStream_t upload_stream, kvx_plan_t** out);
// Bytes of a plan's device work list, and its copy into device memory `buf`
// on stream `s` (which also points the plan's device fields into `buf`).
size_t worklist_bytes(const kvx_plan_t* plan);
int worklist_copy(kvx_plan_t* plan, char* buf, hipStream_t s);

// Validate one (plan, layer) pair of a batched push (pair index i for the
// message): a device plan with a push work list and a layer in range.
int check_push_pair(const kvx_plan_t* plan, int32_t layer, const char* fn, int32_t i);

// Enqueue the pushes of already validated pairs on `stream` (after each
// plan's upload), batched into as few launches as kvx_push_many uses; no
// ready wait.  `started` / `finished` (nullable) receive the first launch's
// start and the last launch's end timestamps; *launches (nullable) grows by
// the kernel launches enqueued.
int push_batch(const kvx_plan_t* const* plans, const int32_t* layers, int32_t n, hipStream_t stream,
               hipEvent_t started = nullptr, hipEvent_t finished = nullptr, int64_t* launches = nullptr);

// One layer's head-slice write (what kvx_copy_heads copies).
struct HeadsWrite {
  const kvx_plan_t* plan;
  int32_t layer, src_head0, dst_head0, num_heads;
};
// Validate a head-slice write as kvx_copy_heads does.
int check_heads_write(const HeadsWrite& w, const char* fn);
// Enqueue already validated head-slice writes on `stream` (after each plan's
// upload): consecutive writes of one plan and head slice share launches of
// up to 32 layers, as in kvx_copy_heads_layers.  Every launch records its
// end into `finished` (nullable; the last one wins); *launches (nullable)
// grows by the kernel launches enqueued.
int heads_batch(const HeadsWrite* writes, int32_t n, hipStream_t stream, hipEvent_t finished = nullptr,
                int64_t* launches = nullptr);

}  // namespace kvx
