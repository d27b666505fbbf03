// specverify.hip -- host side of libspecverify: the C ABI declared in
// include/specverify.h (argument validation, workspace layout, dtype and
// alignment dispatch, launches, optional kernel timing).
//
// Scheme: "Accelerating Sonar through speculation" (Perplexity, 2025); the
// entry points correspond to its sections "Target-Draft" (chain
// verification with sampling), "Speculative decoding" (greedy matching),
// "EAGLE" (tree verification, greedy and sampled) and "MTP Schedule for a
// Single Token" (the device-side commit).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cstdint>
#include <tuple>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "specverify.h"
#include "sv_kernels.hpp"

// The workspace of sv_verify_chain_static: one copy per GPU, held until the
// process ends.  Host code uses the device address that hipGetSymbolAddress
// returns for the current device (see static_workspace), never the array's
// name.
static __device__ __align__(256) unsigned char scratch[SV_STATIC_WORKSPACE_BYTES];

namespace {

using sv::Partial;
using sv::SeqInfo;

// Vectors of 16 bytes per lane per tile in the passes over every row.
constexpr int kU = 8;

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int elem_bytes(sv_dtype dt) { return dt == SV_BF16 ? 2 : 4; }

bool valid_dtype(sv_dtype dt) { return dt == SV_F32 || dt == SV_BF16; }

// Tiles per row: NV = ceil(V / VE) vectors of 16 bytes, 64 * u vectors per tile.
int64_t tiles_per_row(int V, sv_dtype dt, int u = kU) {
    const int64_t ve = 16 / elem_bytes(dt);
    const int64_t nv = (V + ve - 1) / ve;
    return (nv + 64 * u - 1) / (64 * u);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Blocks of kBlock threads for `waves` independent wave64 tiles.
int64_t blocks_for_waves(int64_t waves) { return (waves + sv::kWavesPerBlock - 1) / sv::kWavesPerBlock; }

constexpr int64_t kMaxGrid = 0x7fffffff;

// Largest accepted max_depth of the tree entry points (output rows of
// max_depth + 1 entries; no tree of SV_MAX_TREE_NODES nodes is deeper than
// SV_MAX_TREE_NODES - 1, so this only guards the arithmetic).
constexpr int kMaxDepth = 1 << 24;

// ---------------------------------------------------------------- workspace layouts ---

// Segments (64 vectors of 16 bytes) per row, and the final draw's chunks of
// kSegPerChunk segments.
int64_t segments_per_row(int V, sv_dtype dt) {
    const int64_t ve = 16 / elem_bytes(dt);
    return ((V + ve - 1) / ve + 63) / 64;
}
int64_t final_chunks(int V, sv_dtype dt) {
    return (segments_per_row(V, dt) + sv::kSegPerChunk - 1) / sv::kSegPerChunk;
}

// Small chains take one launch, one workgroup per sequence
// (chain_small_kernel): up to kSmallMaxRows sequences whose rows have at
// most kSmallMaxSegs segments and whose 2k + 1 rows hold at most
// kSmallMaxBytes, which one CU streams in about the launches it saves
// (without drafts, below the one-workgroup-per-row draw's batch size).
// Small greedy chains likewise (greedy_small_kernel), when their k + 1 rows
// fit in one tile per wave (at most 128 KiB): the argmax is cheap enough
// that a second round of tiles costs more than the launch saved.
constexpr int kSmallMaxRows = 256;
constexpr int64_t kSmallMaxBytes = 144 * 1024;

// Largest final-draw grid for which every workgroup recomputes its
// sequence's acceptance; beyond it one wave per sequence computes it once.
constexpr int64_t kInlineAcceptMaxBlocks = 2048;

// Chains without accept_prob stream their rows in two phases (positions
// 0 .. max(1, k/4)-1, then, after chain_prefix has flagged the sequences
// that accept all of those, the rest for those sequences only) from this many
// drafts and this many bytes of rows on.  The flag kernel and the second
// launch cost about 6 us: at k = 8 (265 MB, 28% of sequences past position
// 1) the step gains 24%, at k = 4 (131 MB, 56% past position 0) it loses 2%.
constexpr int kChainTwoPhaseMinK = 6;
constexpr int64_t kChainTwoPhaseMinBytes = int64_t(128) << 20;
constexpr int kChainFirstPhaseDiv = 4;
constexpr int kChainRestTilesPerWave = 1;

// Plain sampling (no drafts) runs one workgroup per sequence
// (chain_row_draw_kernel) from this many sequences on, for rows of at most
// kRowDrawMaxSegs segments: one row per CU fills the chip.  Below it a row
// alone on a CU streams too slowly and the two-kernel draw (rows split over
// many workgroups) is faster.  With drafts the draw stays split: a residual
// costs about three times the arithmetic of a bonus draw per element, so one
// sequence per CU leaves the CUs that hold residuals as the kernel's tail.
constexpr int kRowDrawMinRows = 256;

// Chains whose draw recomputes the acceptance in every workgroup stream
// their rows and draw in one launch (chain_fused_kernel) when one wave's
// group_load holds all 2k rows' partials: G lanes per row with G * 2k <= 64,
// at most kBatch partials per lane.
bool fused_fits(int k, int nT) {
    if (2 * k > sv::kWave) return false;
    int G = sv::kWave;
    while (G > 1 && G * 2 * k > sv::kWave) G >>= 1;
    return nT <= sv::kBatch * G;
}

// How many times a drawing workgroup of chain_fused_kernel reads its
// sequence's published partials before computing any still missing itself
// (sv_set_handoff_polls).  About 80 ms of waiting: far beyond any call's
// streaming, so the bound only guarantees that every wait ends.
constexpr int kDefaultHandoffPolls = 1 << 16;
std::atomic<int> g_handoff_polls{kDefaultHandoffPolls};

// The tag of a call's handed-over partials (sv::CallTag): a new 64-bit epoch
// per call, mapped one-to-one onto the two words' halves.  Epoch 0 would map
// to (0, 0), the cleared slots' tag; epoch 1 is the one tag of every call
// made while its stream is captured into a graph (a graph replays its
// arguments), whose slots are therefore cleared first.
std::atomic<uint64_t> g_call_epoch{2};
constexpr uint64_t kCaptureEpoch = 1;

sv::CallTag call_tag(uint64_t e) {
    const uint32_t lo = static_cast<uint32_t>(e);
    return sv::CallTag{lo, static_cast<uint32_t>(e >> 32) ^ (lo * 0x9e3779b9u)};
}

// Whether work issued to `stream` is being captured (or the query fails:
// then the caller takes the path that is right either way).
bool stream_capturing(hipStream_t stream) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
        (void)hipGetLastError();
        return true;
    }
    return cs != hipStreamCaptureStatusNone;
}

// The chain workspace: the per-(row, tile) partials of the 2k streamed rows of
// every sequence, their logits at the draft tokens, the final draw's
// descriptors, segment masses and chunk argmaxes.
struct ChainLayout {
    size_t part, gathered, info, segs, chunkarg, go, total;
};

ChainLayout chain_layout(int B, int k, int V, sv_dtype dt) {
    ChainLayout L{};
    L.part = 0;
    // room for the tagged slots of the one-launch path (chain_fused_kernel)
    L.gathered = align_up(L.part + sizeof(sv::TaggedPartial) * static_cast<size_t>(2) * B * k * tiles_per_row(V, dt));
    L.info = align_up(L.gathered + sizeof(float) * static_cast<size_t>(2) * B * k);
    L.segs = align_up(L.info + sizeof(SeqInfo) * static_cast<size_t>(B));
    L.chunkarg = align_up(L.segs + sizeof(sv::SegMass) * static_cast<size_t>(B) * segments_per_row(V, dt));
    L.go = align_up(L.chunkarg + sizeof(Partial) * static_cast<size_t>(B) * final_chunks(V, dt));
    L.total = align_up(L.go + sizeof(int32_t) * static_cast<size_t>(B));
    return L;
}

// The sampled-tree workspace: partials of every node's two rows, the
// children's gathered logits, the walk's double-buffered state and pass
// partial sums (P slices per sequence), the final draw's segment masses,
// every node's combined normalisers and the per-segment statistics of the
// leaf a walk ends at.
struct TreeSampledLayout {
    int P;
    size_t part, tg, dg, state, z, tsegs, norm, leaf, total;
};

TreeSampledLayout tree_sampled_layout(int B, int N, int V, sv_dtype dt) {
    TreeSampledLayout L{};
    const int64_t nseg = segments_per_row(V, dt);
    // slices of at least four segments, about 1024 workgroups per round
    const int64_t want = (1024 + std::max(B, 1) - 1) / std::max(B, 1);
    L.P = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(want, (nseg + 3) / 4)));
    const size_t bn = static_cast<size_t>(B) * N;
    L.part = 0;
    L.tg = align_up(sizeof(Partial) * 2 * bn * tiles_per_row(V, dt));
    L.dg = align_up(L.tg + sizeof(float) * bn);
    L.state = align_up(L.dg + sizeof(float) * bn);
    L.z = align_up(L.state + sizeof(sv::WalkState) * 2 * static_cast<size_t>(B));
    L.tsegs = align_up(L.z + sizeof(double) * 4 * 2 * static_cast<size_t>(B) * L.P);
    L.norm = align_up(L.tsegs + sizeof(float) * static_cast<size_t>(B) * nseg);
    L.leaf = align_up(L.norm + sizeof(sv::NodeNorm) * bn);
    L.total = align_up(L.leaf + sizeof(Partial) * static_cast<size_t>(B) * nseg);
    return L;
}

// The greedy-tree workspace: the partials of every node's row, then the
// second phase's node lists and their lengths.
struct TreeLayout {
    size_t part, list, count, slots, total;
};

TreeLayout tree_layout(int B, int N, int V, sv_dtype dt) {
    TreeLayout L{};
    L.part = 0;
    L.list = align_up(sizeof(Partial) * static_cast<size_t>(B) * N * tiles_per_row(V, dt));
    L.count = align_up(L.list + sizeof(int32_t) * static_cast<size_t>(B) * N);
    // the root rows' tagged partials of tree_root_plan_kernel
    L.slots = align_up(L.count + sizeof(int32_t) * static_cast<size_t>(B));
    L.total = align_up(L.slots + sizeof(sv::TaggedPartial) * static_cast<size_t>(B) * tiles_per_row(V, dt));
    return L;
}

// ---------------------------------------------------------------- kernel timing ---

struct ProfSlot {
    std::string name;
    hipEvent_t start = nullptr, stop = nullptr;
    bool used = false;
};

struct Profiler {
    std::mutex mu;
    bool on = false;
    std::vector<ProfSlot> slots;
    size_t next = 0;
} g_prof;

// Launch `kernel` on `stream`.  While profiling, the launch carries an event
// pair that the runtime records at the dispatch's own start and end
// (hipExtLaunchKernel), so the measured time is the kernel's execution alone.
template <typename... KArgs, typename... Args>
sv_status launch(const char* name, void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
                 Args... args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
    std::tuple<KArgs...> params(static_cast<KArgs>(args)...);
    void* argv[sizeof...(KArgs)];
    std::apply([&argv](auto&... p) {
        size_t i = 0;
        ((argv[i++] = static_cast<void*>(&p)), ...);
    }, params);
    ProfSlot* slot = nullptr;
    if (g_prof.on) {
        std::lock_guard<std::mutex> lk(g_prof.mu);
        if (g_prof.next < g_prof.slots.size()) slot = &g_prof.slots[g_prof.next++];
    }
    // without profiling, the plain launch (the form HIP graph capture records)
    const hipError_t err =
        slot ? hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0, stream, slot->start,
                                  slot->stop, 0)
             : hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0, stream);
    if (err != hipSuccess) {
        (void)hipGetLastError();
        return SV_ERR_HIP;
    }
    if (slot) {
        slot->name = name;
        slot->used = true;
    }
    return SV_OK;
}

// ---------------------------------------------------------------- dispatch ---

// The tag of a launch that hands partials between its workgroups in tagged
// slots (sv::CallTag): a new epoch per call, or, while the stream is being
// captured, the one capture epoch after a launch that clears the slots.
sv_status handover_tag(hipStream_t stream, sv::TaggedPartial* slots, int64_t nslots, sv::CallTag& tag) {
    uint64_t epoch = kCaptureEpoch;
    if (stream_capturing(stream)) {
        const sv_status st = launch("clear_slots", sv::clear_slots_kernel,
                                    dim3(static_cast<unsigned>((nslots + sv::kBlock - 1) / sv::kBlock)),
                                    dim3(sv::kBlock), stream, slots, nslots);
        if (st != SV_OK) return st;
    } else {
        epoch = g_call_epoch.fetch_add(1, std::memory_order_relaxed);
    }
    tag = call_tag(epoch);
    return SV_OK;
}

template <int DT, bool VEC>
sv_status run_chain(int B, int k, int V, const int32_t* tokens, const void* draft, const void* target,
                    const float* temperature, const float* uniforms, int32_t* accepted_len, int32_t* emitted,
                    float* accept_prob, char* ws, const ChainLayout& L, int nT, int nchunk,
                    hipStream_t stream) {
    auto* part = reinterpret_cast<Partial*>(ws + L.part);
    auto* gathered = reinterpret_cast<float*>(ws + L.gathered);
    auto* info = reinterpret_cast<SeqInfo*>(ws + L.info);
    auto* segs = reinterpret_cast<sv::SegMass*>(ws + L.segs);
    auto* chunkarg = reinterpret_cast<Partial*>(ws + L.chunkarg);
    sv_status st;
    if (B <= kSmallMaxRows && (k > 0 || B < kRowDrawMinRows) &&
        segments_per_row(V, static_cast<sv_dtype>(DT)) <= sv::kSmallMaxSegs &&
        static_cast<int64_t>(2 * k) * nT <= sv::kSmallMaxParts &&
        static_cast<int64_t>(2 * k + 1) * V * sv::Elem<DT>::bytes <= kSmallMaxBytes) {
        return launch("chain_small", sv::chain_small_kernel<DT, VEC, kU>, dim3(static_cast<unsigned>(B)),
                      dim3(sv::kSmallBlock), stream, tokens, draft, target, temperature, uniforms, k, V, nT,
                      accepted_len, emitted, accept_prob);
    }
    const int64_t fin_blocks = static_cast<int64_t>(B) * nchunk;
    const int acc = k == 0 ? sv::kAcceptNone
                           : (fin_blocks <= kInlineAcceptMaxBlocks ? sv::kAcceptInline : sv::kAcceptRead);
    // Without accept_prob a sequence's rows after its first rejection are
    // never needed: large chains stream positions 0 .. s-1 first, then the
    // rest only for sequences that accept all of them.
    const int64_t rows_bytes = static_cast<int64_t>(2) * B * k * V * sv::Elem<DT>::bytes;
    const int groups = static_cast<int>(blocks_for_waves(nT));
    const int s = k > 0 && accept_prob == nullptr && k >= kChainTwoPhaseMinK && rows_bytes >= kChainTwoPhaseMinBytes &&
                          static_cast<int64_t>(B) * 2 * k * groups <= kMaxGrid
                      ? std::max(1, k / kChainFirstPhaseDiv)
                      : k;
    auto* segs_c = static_cast<const sv::SegMass*>(segs);
    if (k > 0 && s == k && acc == sv::kAcceptInline && fused_fits(k, nT)) {
        // the rows and the draw in one launch, the partials handed over in
        // slots tagged for this call
        auto* slots = reinterpret_cast<sv::TaggedPartial*>(ws + L.part);
        const int64_t nslots = static_cast<int64_t>(2) * B * k * nT;
        sv::CallTag tag;
        if ((st = handover_tag(stream, slots, nslots, tag)) != SV_OK) return st;
        const int64_t row_blocks = blocks_for_waves(nslots);
        st = launch("chain_fused", sv::chain_fused_kernel<DT, VEC, kU>, dim3(static_cast<unsigned>(row_blocks + fin_blocks)),
                    dim3(sv::kFinBlock), stream, tokens, draft, target, temperature, uniforms, B, k, V, nT, row_blocks,
                    nchunk, g_handoff_polls.load(std::memory_order_relaxed), slots, tag, accepted_len,
                    emitted, accept_prob, info, segs, chunkarg);
        if (st != SV_OK) return st;
        return launch("chain_final_pick", sv::chain_final_pick_kernel<DT, VEC>, dim3(B), dim3(sv::kPickBlock), stream,
                      draft, target, k, V, nchunk, static_cast<const SeqInfo*>(info), segs_c,
                      static_cast<const Partial*>(chunkarg), emitted);
    }
    if (k > 0) {
        const int64_t blocks = blocks_for_waves(static_cast<int64_t>(2) * B * s * nT);
        st = launch("chain_rowstats", sv::chain_rowstats_kernel<DT, VEC, kU>, dim3(static_cast<unsigned>(blocks)),
                    dim3(sv::kBlock), stream, target, draft, temperature, tokens, B, k, 0, s, V, nT, part, gathered);
        if (st != SV_OK) return st;
        if (s < k) {
            auto* go = reinterpret_cast<int32_t*>(ws + L.go);
            st = launch("chain_prefix", sv::chain_prefix_kernel<DT>,
                        dim3(static_cast<unsigned>((B + sv::kAccWaves - 1) / sv::kAccWaves)),
                        dim3(sv::kAccWaves * sv::kWave), stream, tokens, temperature, uniforms, B, k, s, V, nT,
                        static_cast<const Partial*>(part), static_cast<const float*>(gathered), go);
            if (st != SV_OK) return st;
            const int tpw = kChainRestTilesPerWave;
            const int rest_groups = (nT + sv::kWavesPerBlock * tpw - 1) / (sv::kWavesPerBlock * tpw);
            st = launch("chain_rowstats_rest", sv::chain_rowstats_rest_kernel<DT, VEC, kU>,
                        dim3(static_cast<unsigned>(static_cast<int64_t>(B) * 2 * (k - s) * rest_groups)),
                        dim3(sv::kBlock), stream, target, draft, temperature, tokens, static_cast<const int32_t*>(go),
                        B, k, s, V, nT, rest_groups, tpw, part, gathered);
            if (st != SV_OK) return st;
        }
    }
    if (k == 0 && B >= kRowDrawMinRows && segments_per_row(V, static_cast<sv_dtype>(DT)) <= sv::kRowDrawMaxSegs) {
        return launch("chain_row_draw", sv::chain_row_draw_kernel<DT, VEC>, dim3(static_cast<unsigned>(B)),
                      dim3(sv::kRowDrawBlock), stream, target, temperature, uniforms, V, accepted_len, emitted);
    }
    if (acc == sv::kAcceptRead) {
        const unsigned acc_blocks = static_cast<unsigned>((B + sv::kAccWaves - 1) / sv::kAccWaves);
        st = launch("chain_accept", sv::chain_accept_kernel<DT>, dim3(acc_blocks), dim3(sv::kAccWaves * sv::kWave),
                    stream, tokens, temperature, uniforms, B, k, V, nT, static_cast<const Partial*>(part),
                    static_cast<const float*>(gathered), accepted_len, emitted, accept_prob, info);
        if (st != SV_OK) return st;
    }
    auto final_part = acc == sv::kAcceptNone     ? sv::chain_final_part_kernel<DT, VEC, sv::kAcceptNone>
                      : acc == sv::kAcceptInline ? sv::chain_final_part_kernel<DT, VEC, sv::kAcceptInline>
                                                 : sv::chain_final_part_kernel<DT, VEC, sv::kAcceptRead>;
    st = launch("chain_final_part", final_part, dim3(static_cast<unsigned>(fin_blocks)), dim3(sv::kFinBlock), stream,
                tokens, draft, target, temperature, uniforms, B, k, V, nT, static_cast<const Partial*>(part),
                static_cast<const float*>(gathered), nchunk, accepted_len, emitted, accept_prob, info, segs,
                chunkarg);
    if (st != SV_OK) return st;
    return launch("chain_final_pick", sv::chain_final_pick_kernel<DT, VEC>, dim3(B), dim3(sv::kPickBlock), stream, draft,
                  target, k, V, nchunk, static_cast<const SeqInfo*>(info), segs_c, static_cast<const Partial*>(chunkarg),
                  emitted);
}

template <int DT, bool VEC>
sv_status run_argmax_rows(const void* logits, int64_t nrows, int V, int nT, Partial* part, hipStream_t stream) {
    const int64_t blocks = blocks_for_waves(nrows * nT);
    return launch("argmax_rows", sv::argmax_rows_kernel<DT, VEC, kU>, dim3(static_cast<unsigned>(blocks)),
                  dim3(sv::kBlock), stream, logits, nrows, V, nT, part);
}

sv_status argmax_rows(sv_dtype dt, bool vec, const void* logits, int64_t nrows, int V, int nT, Partial* part,
                      hipStream_t stream) {
    if (dt == SV_BF16)
        return vec ? run_argmax_rows<SV_BF16, true>(logits, nrows, V, nT, part, stream)
                   : run_argmax_rows<SV_BF16, false>(logits, nrows, V, nT, part, stream);
    return vec ? run_argmax_rows<SV_F32, true>(logits, nrows, V, nT, part, stream)
               : run_argmax_rows<SV_F32, false>(logits, nrows, V, nT, part, stream);
}

// Tiles per wave in the second phase of greedy verification: fewer
// workgroups, each checking its sequence once for more tiles.
constexpr int kGreedyRestTilesPerWave = 2;

// The greedy rows' launches (greedy_rows_kernel): one workgroup per
// (sequence, row, group of tiles).
template <int DT, bool VEC, bool CHECK>
sv_status run_greedy_rows(const void* logits, const int32_t* tokens, int B, int k, int V, int nT, int nrows, int j0,
                          Partial* part, hipStream_t stream) {
    constexpr int tpw = CHECK ? kGreedyRestTilesPerWave : 1;
    const int groups = (nT + sv::kWavesPerBlock * tpw - 1) / (sv::kWavesPerBlock * tpw);
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(B) * nrows * groups));
    if constexpr (CHECK)
        return launch("greedy_rows_rest", sv::greedy_rows_rest_kernel<DT, VEC, kU, tpw>, grid, dim3(sv::kBlock),
                      stream, logits, tokens, k, V, nT, groups, nrows, j0, part);
    else
        return launch("greedy_rows", sv::greedy_rows_kernel<DT, VEC, kU>, grid, dim3(sv::kBlock), stream, logits,
                      tokens, k, V, nT, groups, nrows, j0, part);
}

// Both phases of a two-phase greedy chain in one launch (greedy_fused_kernel).
template <int DT, bool VEC>
sv_status run_greedy_fused(const void* logits, const int32_t* tokens, int B, int k, int V, int nT, int s,
                           sv::TaggedPartial* slots, sv::CallTag tag, Partial* part, hipStream_t stream) {
    constexpr int tpw = kGreedyRestTilesPerWave;
    const int groups1 = (nT + sv::kWavesPerBlock - 1) / sv::kWavesPerBlock;
    const int groups2 = (nT + sv::kWavesPerBlock * tpw - 1) / (sv::kWavesPerBlock * tpw);
    const int64_t p1_blocks = static_cast<int64_t>(B) * s * groups1;
    const int64_t blocks = p1_blocks + static_cast<int64_t>(B) * (k + 1 - s) * groups2;
    return launch("greedy_fused", sv::greedy_fused_kernel<DT, VEC, kU, tpw>, dim3(static_cast<unsigned>(blocks)),
                  dim3(sv::kBlock), stream, logits, tokens, k, V, nT, s, groups1, groups2, p1_blocks, slots, tag,
                  g_handoff_polls.load(std::memory_order_relaxed), part);
}

sv_status greedy_fused(sv_dtype dt, bool vec, const void* logits, const int32_t* tokens, int B, int k, int V, int nT,
                       int s, sv::TaggedPartial* slots, sv::CallTag tag, Partial* part, hipStream_t stream) {
    if (dt == SV_BF16)
        return vec ? run_greedy_fused<SV_BF16, true>(logits, tokens, B, k, V, nT, s, slots, tag, part, stream)
                   : run_greedy_fused<SV_BF16, false>(logits, tokens, B, k, V, nT, s, slots, tag, part, stream);
    return vec ? run_greedy_fused<SV_F32, true>(logits, tokens, B, k, V, nT, s, slots, tag, part, stream)
               : run_greedy_fused<SV_F32, false>(logits, tokens, B, k, V, nT, s, slots, tag, part, stream);
}

// Whether the first s rows' partials of a sequence fit one wave's group_load
// (the second phase's check in greedy_fused_kernel reads them as published).
bool greedy_fused_fits(int s, int nT) {
    if (s > sv::kWave) return false;
    int G = sv::kWave;
    while (G > 1 && G * s > sv::kWave) G >>= 1;
    return nT <= sv::kBatch * G;
}

sv_status greedy_rows(sv_dtype dt, bool vec, bool check, const void* logits, const int32_t* tokens, int B, int k, int V,
                      int nT, int j0, int nrows, Partial* part, hipStream_t stream) {
    if (dt == SV_BF16) {
        if (vec)
            return check ? run_greedy_rows<SV_BF16, true, true>(logits, tokens, B, k, V, nT, nrows, j0, part, stream)
                         : run_greedy_rows<SV_BF16, true, false>(logits, tokens, B, k, V, nT, nrows, j0, part, stream);
        return check ? run_greedy_rows<SV_BF16, false, true>(logits, tokens, B, k, V, nT, nrows, j0, part, stream)
                     : run_greedy_rows<SV_BF16, false, false>(logits, tokens, B, k, V, nT, nrows, j0, part, stream);
    }
    if (vec)
        return check ? run_greedy_rows<SV_F32, true, true>(logits, tokens, B, k, V, nT, nrows, j0, part, stream)
                     : run_greedy_rows<SV_F32, true, false>(logits, tokens, B, k, V, nT, nrows, j0, part, stream);
    return check ? run_greedy_rows<SV_F32, false, true>(logits, tokens, B, k, V, nT, nrows, j0, part, stream)
                 : run_greedy_rows<SV_F32, false, false>(logits, tokens, B, k, V, nT, nrows, j0, part, stream);
}

// Greedy trees are streamed in two phases (root rows, then the rows below
// an accepted depth-1 node) from this size on.  The two extra launches cost
// about 8 us: on random trees of 64 nodes at a 0.6 match rate the two phases
// lose 2.8 us at 66 MB of rows and gain 6.2 us at 131 MB.
constexpr int64_t kTreeTwoPhaseMinBytes = int64_t(96) << 20;
// ... and in three (root rows, depths 1-2, depths 3 and more) from this size
// and this many nodes on: the third phase pays where many nodes lie at depth
// 3 and more, which the node count stands in for (the tree is on the device).
// Measured on random trees at a 0.6 match rate: 64 nodes gain 2 us at 263 MB
// and 13 us at 525 MB; 16 and 26 nodes lose 1-2.4 us at 253-263 MB.
constexpr int64_t kTreeThreePhaseMinBytes = int64_t(192) << 20;
constexpr int kTreeThreePhaseMinNodes = 48;

template <int DT, bool VEC>
sv_status run_tree_two_phase(const void* logits, const int32_t* tokens, const int32_t* parent, int parent_stride,
                             int B, int N, int V, int nT, bool three, Partial* part, int32_t* list, int32_t* count,
                             sv::TaggedPartial* slots, hipStream_t stream) {
    const int groups = static_cast<int>(blocks_for_waves(nT));
    // depth ranges of the later phases: [1, inf), or [1, 2] then [3, inf)
    const int ranges[2][2] = {{1, three ? 2 : INT_MAX}, {3, INT_MAX}};
    // trees of at most kBlock nodes: the root rows and the first plan in one
    // launch, the root's partials handed over in slots tagged for this call
    const bool root_plan = N <= sv::kBlock;
    sv_status st;
    if (root_plan) {
        sv::CallTag tag;
        if ((st = handover_tag(stream, slots, static_cast<int64_t>(B) * nT, tag)) != SV_OK) return st;
        const int64_t root_blocks = static_cast<int64_t>(B) * groups;
        st = launch("tree_root_plan", sv::tree_root_plan_kernel<DT, VEC, kU>,
                    dim3(static_cast<unsigned>(root_blocks + B)), dim3(sv::kBlock), stream, logits, tokens, parent,
                    parent_stride, N, V, nT, groups, root_blocks, slots, tag,
                    g_handoff_polls.load(std::memory_order_relaxed), ranges[0][1], part, list, count);
    } else {
        st = launch("tree_root_rows", sv::tree_root_rows_kernel<DT, VEC, kU>,
                    dim3(static_cast<unsigned>(static_cast<int64_t>(B) * groups)), dim3(sv::kBlock), stream, logits, N,
                    V, nT, groups, part);
    }
    if (st != SV_OK) return st;
    const int nodes_threads = (N + sv::kWave - 1) / sv::kWave * sv::kWave;
    for (int ph = 0; ph < (three ? 2 : 1); ++ph) {
        // the root's children alone need one wave per node; later ranges combine every row over at least 256 threads
        const int threads = ph == 0 ? nodes_threads : std::max(256, nodes_threads);
        if (ph > 0 || !root_plan) {
            st = launch("tree_plan", sv::tree_plan_kernel, dim3(B), dim3(threads), stream, tokens, parent,
                        parent_stride, N, nT, static_cast<const Partial*>(part), ranges[ph][0], ranges[ph][1], list,
                        count);
            if (st != SV_OK) return st;
        }
        st = launch("tree_rows_rest", sv::tree_rows_rest_kernel<DT, VEC, kU>,
                    dim3(static_cast<unsigned>(static_cast<int64_t>(B) * (N - 1) * groups)), dim3(sv::kBlock), stream,
                    logits, N, V, nT, groups, static_cast<const int32_t*>(list), static_cast<const int32_t*>(count),
                    part);
        if (st != SV_OK) return st;
    }
    return SV_OK;
}

sv_status tree_two_phase(sv_dtype dt, bool vec, const void* logits, const int32_t* tokens, const int32_t* parent,
                         int parent_stride, int B, int N, int V, int nT, bool three, Partial* part, int32_t* list,
                         int32_t* count, sv::TaggedPartial* slots, hipStream_t stream) {
    if (dt == SV_BF16)
        return vec ? run_tree_two_phase<SV_BF16, true>(logits, tokens, parent, parent_stride, B, N, V, nT, three, part,
                                                       list, count, slots, stream)
                   : run_tree_two_phase<SV_BF16, false>(logits, tokens, parent, parent_stride, B, N, V, nT, three,
                                                        part, list, count, slots, stream);
    return vec ? run_tree_two_phase<SV_F32, true>(logits, tokens, parent, parent_stride, B, N, V, nT, three, part,
                                                  list, count, slots, stream)
               : run_tree_two_phase<SV_F32, false>(logits, tokens, parent, parent_stride, B, N, V, nT, three, part,
                                                   list, count, slots, stream);
}

// The greedy workspace: the partials of every row, then the tagged slots of
// the first phase's rows (at most (k + 1) / 2 per sequence) that
// greedy_fused_kernel hands between its phases.
size_t greedy_slots_offset(int B, int k, int V, sv_dtype dt) {
    return align_up(sizeof(Partial) * static_cast<size_t>(B) * (k + 1) * tiles_per_row(V, dt));
}

// Greedy verification streams its rows in two phases only from this size on.
// The second phase costs about 5 us beyond the rows it streams (a dependent
// launch, the check's round trip, workgroups that exit): at a 0.8 match rate
// and k = 4 or 5 it loses up to 200 MB of rows and gains 12% at 394 MB.
constexpr int64_t kGreedyTwoPhaseMinBytes = int64_t(256) << 20;

// Checks shared by the entry points: a positive vocabulary within limits and a
// grid that fits the launch limits for `rows` rows.
sv_status check_rows(int64_t rows, int V, sv_dtype dt) {
    if (V < 1 || !valid_dtype(dt)) return SV_ERR_INVALID_ARGUMENT;
    if (V > SV_MAX_VOCAB) return SV_ERR_UNSUPPORTED;
    const int64_t nT = tiles_per_row(V, dt);
    if (rows > 0 && blocks_for_waves(rows * nT) > kMaxGrid) return SV_ERR_UNSUPPORTED;
    return SV_OK;
}

sv_status check_workspace(void* ws, size_t have, size_t need) {
    if (have < need) return SV_ERR_WORKSPACE_TOO_SMALL;
    if (need > 0 && (ws == nullptr || !aligned16(ws))) return SV_ERR_INVALID_ARGUMENT;
    return SV_OK;
}

// ---------------------------------------------------------------- static workspace ---

struct StaticWorkspace {
    std::mutex mu;
    std::vector<void*> ptr;  // per device id, looked up on the first call there
} g_static_ws;

sv_status static_workspace(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return SV_ERR_HIP;
    }
    std::lock_guard<std::mutex> lk(g_static_ws.mu);
    if (static_cast<size_t>(dev) >= g_static_ws.ptr.size()) g_static_ws.ptr.resize(dev + 1, nullptr);
    if (g_static_ws.ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return SV_ERR_HIP;
        }
        g_static_ws.ptr[dev] = p;
    }
    *out = g_static_ws.ptr[dev];
    return SV_OK;
}

}  // namespace

extern "C" {

int sv_version(void) { return 100; }

int sv_set_handoff_polls(int polls) {
    return g_handoff_polls.exchange(polls < 0 ? kDefaultHandoffPolls : polls, std::memory_order_relaxed);
}

const char* sv_status_string(sv_status s) {
    switch (s) {
        case SV_OK: return "SV_OK";
        case SV_ERR_INVALID_ARGUMENT: return "SV_ERR_INVALID_ARGUMENT: invalid argument";
        case SV_ERR_WORKSPACE_TOO_SMALL: return "SV_ERR_WORKSPACE_TOO_SMALL: workspace smaller than required";
        case SV_ERR_UNSUPPORTED: return "SV_ERR_UNSUPPORTED: size beyond the supported limits";
        case SV_ERR_HIP: return "SV_ERR_HIP: HIP runtime or launch failure";
    }
    return "unknown sv_status";
}

size_t sv_chain_workspace_bytes(int B, int k, int V, sv_dtype dt) {
    if (B < 0 || k < 0 || k > SV_MAX_DRAFTS || V < 1 || V > SV_MAX_VOCAB || !valid_dtype(dt)) return 0;
    return chain_layout(B, k, V, dt).total;
}

size_t sv_greedy_workspace_bytes(int B, int k, int V, sv_dtype dt) {
    if (B < 0 || k < 0 || k > SV_MAX_DRAFTS || V < 1 || V > SV_MAX_VOCAB || !valid_dtype(dt)) return 0;
    return greedy_slots_offset(B, k, V, dt) +
           align_up(sizeof(sv::TaggedPartial) * static_cast<size_t>(B) * ((k + 1) / 2) * tiles_per_row(V, dt));
}

size_t sv_tree_workspace_bytes(int B, int N, int V, sv_dtype dt) {
    if (B < 0 || N < 1 || N > SV_MAX_TREE_NODES || V < 1 || V > SV_MAX_VOCAB || !valid_dtype(dt)) return 0;
    return tree_layout(B, N, V, dt).total;
}

size_t sv_tree_sampled_workspace_bytes(int B, int N, int V, sv_dtype dt) {
    if (B < 0 || N < 1 || N > SV_MAX_TREE_NODES || V < 1 || V > SV_MAX_VOCAB || !valid_dtype(dt)) return 0;
    return tree_sampled_layout(B, N, V, dt).total;
}

sv_status sv_verify_chain(int B, int k, int V, sv_dtype dt, const int32_t* draft_tokens, const void* draft_logits,
                          const void* target_logits, const float* temperature, const float* uniforms,
                          int32_t* accepted_len, int32_t* emitted, float* accept_prob, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
    if (B < 0 || k < 0) return SV_ERR_INVALID_ARGUMENT;
    if (k > SV_MAX_DRAFTS) return SV_ERR_UNSUPPORTED;
    sv_status st = check_rows(static_cast<int64_t>(2) * B * (k + 1), V, dt);
    if (st != SV_OK) return st;
    if (B == 0) return SV_OK;
    if (!target_logits || !temperature || !uniforms || !accepted_len || !emitted) return SV_ERR_INVALID_ARGUMENT;
    if (k > 0 && (!draft_tokens || !draft_logits)) return SV_ERR_INVALID_ARGUMENT;
    const ChainLayout L = chain_layout(B, k, V, dt);
    if ((st = check_workspace(workspace, workspace_bytes, L.total)) != SV_OK) return st;
    const int nT = static_cast<int>(tiles_per_row(V, dt));
    const int nchunk = static_cast<int>(final_chunks(V, dt));
    if (static_cast<int64_t>(B) * nchunk > kMaxGrid) return SV_ERR_UNSUPPORTED;
    const bool vec = (static_cast<int64_t>(V) * elem_bytes(dt)) % 16 == 0 && aligned16(target_logits) &&
                     (k == 0 || aligned16(draft_logits));
    char* ws = static_cast<char*>(workspace);
    if (dt == SV_BF16)
        return vec ? run_chain<SV_BF16, true>(B, k, V, draft_tokens, draft_logits, target_logits, temperature,
                                              uniforms, accepted_len, emitted, accept_prob, ws, L, nT, nchunk, stream)
                   : run_chain<SV_BF16, false>(B, k, V, draft_tokens, draft_logits, target_logits, temperature,
                                               uniforms, accepted_len, emitted, accept_prob, ws, L, nT, nchunk, stream);
    return vec ? run_chain<SV_F32, true>(B, k, V, draft_tokens, draft_logits, target_logits, temperature,
                                         uniforms, accepted_len, emitted, accept_prob, ws, L, nT, nchunk, stream)
               : run_chain<SV_F32, false>(B, k, V, draft_tokens, draft_logits, target_logits, temperature,
                                          uniforms, accepted_len, emitted, accept_prob, ws, L, nT, nchunk, stream);
}

sv_status sv_verify_chain_static(int B, int k, int V, sv_dtype dt, const int32_t* draft_tokens,
                                 const void* draft_logits, const void* target_logits, const float* temperature,
                                 const float* uniforms, int32_t* accepted_len, int32_t* emitted, float* accept_prob,
                                 hipStream_t stream) {
    if (B < 0 || k < 0) return SV_ERR_INVALID_ARGUMENT;
    if (k > SV_MAX_DRAFTS) return SV_ERR_UNSUPPORTED;
    sv_status st = check_rows(static_cast<int64_t>(2) * B * (k + 1), V, dt);
    if (st != SV_OK) return st;
    if (B == 0) return SV_OK;
    if (!target_logits || !temperature || !uniforms || !accepted_len || !emitted) return SV_ERR_INVALID_ARGUMENT;
    if (k > 0 && (!draft_tokens || !draft_logits)) return SV_ERR_INVALID_ARGUMENT;
    if (chain_layout(B, k, V, dt).total > SV_STATIC_WORKSPACE_BYTES) return SV_ERR_WORKSPACE_TOO_SMALL;
    void* ws = nullptr;
    if ((st = static_workspace(&ws)) != SV_OK) return st;
    return sv_verify_chain(B, k, V, dt, draft_tokens, draft_logits, target_logits, temperature, uniforms,
                           accepted_len, emitted, accept_prob, ws, SV_STATIC_WORKSPACE_BYTES, stream);
}

sv_status sv_verify_greedy(int B, int k, int V, sv_dtype dt, const int32_t* draft_tokens, const void* target_logits,
                           int32_t* accepted_len, int32_t* emitted, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
    if (B < 0 || k < 0) return SV_ERR_INVALID_ARGUMENT;
    if (k > SV_MAX_DRAFTS) return SV_ERR_UNSUPPORTED;
    sv_status st = check_rows(static_cast<int64_t>(B) * (k + 1), V, dt);
    if (st != SV_OK) return st;
    if (B == 0) return SV_OK;
    if (!target_logits || !accepted_len || !emitted || (k > 0 && !draft_tokens)) return SV_ERR_INVALID_ARGUMENT;
    if ((st = check_workspace(workspace, workspace_bytes, sv_greedy_workspace_bytes(B, k, V, dt))) != SV_OK)
        return st;
    const int nT = static_cast<int>(tiles_per_row(V, dt));
    if (static_cast<int64_t>(B) * (k + 1) * blocks_for_waves(nT) > kMaxGrid) return SV_ERR_UNSUPPORTED;
    const bool vec = (static_cast<int64_t>(V) * elem_bytes(dt)) % 16 == 0 && aligned16(target_logits);
    auto* part = static_cast<Partial*>(workspace);
    if (B <= kSmallMaxRows && static_cast<int64_t>(k + 1) * nT <= sv::kSmallWaves) {
        auto small = dt == SV_BF16 ? (vec ? sv::greedy_small_kernel<SV_BF16, true, kU>
                                          : sv::greedy_small_kernel<SV_BF16, false, kU>)
                                   : (vec ? sv::greedy_small_kernel<SV_F32, true, kU>
                                          : sv::greedy_small_kernel<SV_F32, false, kU>);
        return launch("greedy_small", small, dim3(static_cast<unsigned>(B)), dim3(sv::kSmallBlock), stream,
                      target_logits, draft_tokens, k, V, nT, accepted_len, emitted);
    }
    // Two phases when the rows they may skip outweigh a dependent launch: rows
    // 0 .. s-1 first, the rest only for sequences whose first s drafts match.
    const int64_t bytes = static_cast<int64_t>(B) * (k + 1) * V * elem_bytes(dt);
    const int s = (k >= 1 && bytes >= kGreedyTwoPhaseMinBytes) ? (k + 1) / 2 : k + 1;
    if (s < k + 1 && greedy_fused_fits(s, nT)) {
        // both phases in one launch, the first phase's partials handed over
        // in slots tagged for this call
        auto* slots = reinterpret_cast<sv::TaggedPartial*>(static_cast<char*>(workspace) +
                                                           greedy_slots_offset(B, k, V, dt));
        sv::CallTag tag;
        if ((st = handover_tag(stream, slots, static_cast<int64_t>(B) * s * nT, tag)) != SV_OK) return st;
        if ((st = greedy_fused(dt, vec, target_logits, draft_tokens, B, k, V, nT, s, slots, tag, part, stream)) !=
            SV_OK)
            return st;
    } else {
        if ((st = greedy_rows(dt, vec, false, target_logits, draft_tokens, B, k, V, nT, 0, s, part, stream)) != SV_OK)
            return st;
        if (s < k + 1 && (st = greedy_rows(dt, vec, true, target_logits, draft_tokens, B, k, V, nT, s, k + 1 - s, part,
                                           stream)) != SV_OK)
            return st;
    }
    return launch("greedy_finalize", sv::greedy_finalize_kernel, dim3(B), dim3(sv::kWave), stream, draft_tokens, k,
                  nT, part, accepted_len, emitted);
}

sv_status sv_verify_tree(int B, int N, int V, sv_dtype dt, const int32_t* node_tokens, const int32_t* parent,
                         int parent_stride, int max_depth, const void* target_logits, int32_t* accepted_len,
                         int32_t* emitted, int32_t* accepted_nodes, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
    if (B < 0 || N < 1 || max_depth < 0 || parent_stride < 0 || (parent_stride != 0 && parent_stride < N))
        return SV_ERR_INVALID_ARGUMENT;
    if (N > SV_MAX_TREE_NODES || max_depth > kMaxDepth) return SV_ERR_UNSUPPORTED;
    sv_status st = check_rows(static_cast<int64_t>(B) * N, V, dt);
    if (st != SV_OK) return st;
    if (B == 0) return SV_OK;
    if (!node_tokens || !parent || !target_logits || !accepted_len || !emitted) return SV_ERR_INVALID_ARGUMENT;
    if ((st = check_workspace(workspace, workspace_bytes, sv_tree_workspace_bytes(B, N, V, dt))) != SV_OK)
        return st;
    const int nT = static_cast<int>(tiles_per_row(V, dt));
    const bool vec = (static_cast<int64_t>(V) * elem_bytes(dt)) % 16 == 0 && aligned16(target_logits);
    const TreeLayout L = tree_layout(B, N, V, dt);
    char* ws = static_cast<char*>(workspace);
    auto* part = reinterpret_cast<Partial*>(ws + L.part);
    const int64_t bytes = static_cast<int64_t>(B) * N * V * elem_bytes(dt);
    if (N > 1 && bytes >= kTreeTwoPhaseMinBytes &&
        static_cast<int64_t>(B) * (N - 1) * blocks_for_waves(nT) <= kMaxGrid) {
        auto* list = reinterpret_cast<int32_t*>(ws + L.list);
        auto* count = reinterpret_cast<int32_t*>(ws + L.count);
        if ((st = tree_two_phase(dt, vec, target_logits, node_tokens, parent, parent_stride, B, N, V, nT,
                                 bytes >= kTreeThreePhaseMinBytes && N >= kTreeThreePhaseMinNodes, part, list,
                                 count, reinterpret_cast<sv::TaggedPartial*>(ws + L.slots), stream)) != SV_OK)
            return st;
    } else if ((st = argmax_rows(dt, vec, target_logits, static_cast<int64_t>(B) * N, V, nT, part, stream)) !=
               SV_OK) {
        return st;
    }
    // one thread per node, and at least 256 so that each node's argmax partials are spread over several lanes
    const int threads = std::max(256, (N + sv::kWave - 1) / sv::kWave * sv::kWave);
    return launch("tree_finalize", sv::tree_finalize_kernel, dim3(B), dim3(threads), stream, node_tokens, parent,
                  parent_stride, N, max_depth, nT, part, accepted_len, emitted, accepted_nodes);
}

// Tiles per wave in the sampled tree's rowstats pass: each wave scans the
// parent array once for two tiles.  One tile took 54 us on 16 trees of 64
// nodes at V = 128256 (bf16), two tiles 51.5, four 52.8.
constexpr int kTreeRowstatsTilesPerWave = 2;

sv_status sv_verify_tree_sampled(int B, int N, int V, sv_dtype dt, const int32_t* node_tokens,
                                 const int32_t* parent, int parent_stride, int max_depth, const void* draft_logits,
                                 const void* target_logits, const float* temperature, const float* uniforms,
                                 int32_t* accepted_len, int32_t* emitted, int32_t* accepted_nodes, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
    if (B < 0 || N < 1 || max_depth < 0 || parent_stride < 0 || (parent_stride != 0 && parent_stride < N))
        return SV_ERR_INVALID_ARGUMENT;
    if (N > SV_MAX_TREE_NODES || max_depth > kMaxDepth) return SV_ERR_UNSUPPORTED;
    sv_status st = check_rows(static_cast<int64_t>(2) * B * N, V, dt);
    if (st != SV_OK) return st;
    if (B == 0) return SV_OK;
    if (!node_tokens || !parent || !draft_logits || !target_logits || !temperature || !uniforms || !accepted_len ||
        !emitted)
        return SV_ERR_INVALID_ARGUMENT;
    if ((st = check_workspace(workspace, workspace_bytes, sv_tree_sampled_workspace_bytes(B, N, V, dt))) != SV_OK)
        return st;
    const int nT = static_cast<int>(tiles_per_row(V, dt));
    const bool vec = (static_cast<int64_t>(V) * elem_bytes(dt)) % 16 == 0 && aligned16(target_logits) &&
                     aligned16(draft_logits);
    const TreeSampledLayout L = tree_sampled_layout(B, N, V, dt);
    if (static_cast<int64_t>(B) * L.P > kMaxGrid) return SV_ERR_UNSUPPORTED;
    char* ws = static_cast<char*>(workspace);
    auto* part = reinterpret_cast<Partial*>(ws + L.part);
    auto* tg = reinterpret_cast<float*>(ws + L.tg);
    auto* dg = reinterpret_cast<float*>(ws + L.dg);
    auto* state = reinterpret_cast<sv::WalkState*>(ws + L.state);
    auto* z = reinterpret_cast<double*>(ws + L.z);
    auto* tsegs = reinterpret_cast<float*>(ws + L.tsegs);
    auto* norm = reinterpret_cast<sv::NodeNorm*>(ws + L.norm);
    auto* leafpart = reinterpret_cast<Partial*>(ws + L.leaf);
    constexpr int tpw = kTreeRowstatsTilesPerWave;
    const unsigned blocks =
        static_cast<unsigned>(blocks_for_waves(static_cast<int64_t>(2) * B * N * ((nT + tpw - 1) / tpw)));
    auto rowstats = dt == SV_BF16 ? (vec ? sv::tree_rowstats_kernel<SV_BF16, true, kU, tpw>
                                         : sv::tree_rowstats_kernel<SV_BF16, false, kU, tpw>)
                                  : (vec ? sv::tree_rowstats_kernel<SV_F32, true, kU, tpw>
                                         : sv::tree_rowstats_kernel<SV_F32, false, kU, tpw>);
    st = launch("tree_rowstats", rowstats, dim3(blocks), dim3(sv::kBlock), stream, target_logits, draft_logits,
                parent, parent_stride, node_tokens, temperature, B, N, V, nT, part, tg, dg);
    if (st != SV_OK) return st;
    auto round = dt == SV_BF16 ? (vec ? sv::tree_round_kernel<SV_BF16, true> : sv::tree_round_kernel<SV_BF16, false>)
                               : (vec ? sv::tree_round_kernel<SV_F32, true> : sv::tree_round_kernel<SV_F32, false>);
    for (int r = 0; r < sv::kWalkRounds; ++r) {
        st = launch("tree_round", round, dim3(static_cast<unsigned>(static_cast<int64_t>(B) * L.P)),
                    dim3(sv::kRoundBlock), stream, node_tokens, parent, parent_stride, N, max_depth, draft_logits,
                    target_logits, temperature, uniforms, B, V, nT, static_cast<const Partial*>(part),
                    static_cast<const float*>(tg), static_cast<const float*>(dg),
                    static_cast<const sv::WalkState*>(state + (r & 1) * B), state + ((r + 1) & 1) * B,
                    static_cast<const double*>(z + static_cast<size_t>(r & 1) * 4 * B * L.P),
                    z + static_cast<size_t>((r + 1) & 1) * 4 * B * L.P, tsegs, norm, leafpart, L.P, r == 0 ? 1 : 0,
                    accepted_len,
                    emitted, accepted_nodes);
        if (st != SV_OK) return st;
    }
    // what the rounds leave: the final draw from masses the last round wrote, or the
    // rest of the walk on one workgroup per sequence, from the last round's state
    auto walk = dt == SV_BF16 ? (vec ? sv::tree_sample_kernel<SV_BF16, true> : sv::tree_sample_kernel<SV_BF16, false>)
                              : (vec ? sv::tree_sample_kernel<SV_F32, true> : sv::tree_sample_kernel<SV_F32, false>);
    return launch("tree_sample", walk, dim3(B), dim3(sv::kWalkBlock), stream, node_tokens, parent, parent_stride, N,
                  max_depth, draft_logits, target_logits, temperature, uniforms, B, V, nT,
                  static_cast<const Partial*>(part), static_cast<const sv::WalkState*>(state + (sv::kWalkRounds & 1) * B),
                  static_cast<const float*>(tsegs), accepted_len, emitted, accepted_nodes);
}

sv_status sv_commit_tokens(int B, int width, const int32_t* accepted_len, const int32_t* emitted, int32_t* seq_len,
                           int32_t* history, int history_stride, int32_t* packed_offsets, int32_t* packed,
                           int32_t* status, hipStream_t stream) {
    if (B < 0 || width < 1 || history_stride < 0) return SV_ERR_INVALID_ARGUMENT;
    if (B > (1 << 24)) return SV_ERR_UNSUPPORTED;
    if (B == 0) return SV_OK;
    if (!accepted_len || !emitted || !seq_len) return SV_ERR_INVALID_ARGUMENT;
    if (static_cast<int64_t>(B) * width > 0x7fffffff) return SV_ERR_UNSUPPORTED;
    return launch("commit_tokens", sv::commit_tokens_kernel, dim3(1), dim3(sv::kCommitBlock), stream, B, width,
                  accepted_len, emitted, seq_len, history, history_stride, packed_offsets, packed, status);
}

sv_status sv_profile_begin(int max_launches) {
    if (max_launches < 0) return SV_ERR_INVALID_ARGUMENT;
    std::lock_guard<std::mutex> lk(g_prof.mu);
    for (auto& s : g_prof.slots) {
        if (s.start) (void)hipEventDestroy(s.start);
        if (s.stop) (void)hipEventDestroy(s.stop);
    }
    g_prof.slots.assign(static_cast<size_t>(max_launches), ProfSlot{});
    for (auto& s : g_prof.slots) {
        if (hipEventCreate(&s.start) != hipSuccess || hipEventCreate(&s.stop) != hipSuccess) {
            g_prof.on = false;
            return SV_ERR_HIP;
        }
    }
    g_prof.next = 0;
    g_prof.on = true;
    return SV_OK;
}

int sv_profile_end(sv_kernel_time* out, int max_out) {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    g_prof.on = false;
    std::vector<sv_kernel_time> agg;
    int rc = 0;
    for (auto& s : g_prof.slots) {
        if (!s.used) continue;
        float ms = 0.f;
        if (hipEventSynchronize(s.stop) != hipSuccess || hipEventElapsedTime(&ms, s.start, s.stop) != hipSuccess) {
            rc = -1;
            continue;
        }
        sv_kernel_time* rec = nullptr;
        for (auto& a : agg)
            if (s.name == a.name) rec = &a;
        if (!rec) {
            agg.push_back(sv_kernel_time{});
            rec = &agg.back();
            std::strncpy(rec->name, s.name.c_str(), sizeof(rec->name) - 1);
        }
        rec->launches += 1;
        rec->total_ms += ms;
    }
    for (auto& s : g_prof.slots) {
        if (s.start) (void)hipEventDestroy(s.start);
        if (s.stop) (void)hipEventDestroy(s.stop);
    }
    g_prof.slots.clear();
    g_prof.next = 0;
    if (rc < 0) return -1;
    const int n = static_cast<int>(agg.size()) < max_out ? static_cast<int>(agg.size()) : max_out;
    if (out)
        for (int i = 0; i < n; ++i) out[i] = agg[i];
    return n;
}

}  // extern "C"
