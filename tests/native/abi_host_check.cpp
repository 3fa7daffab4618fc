// Host-side check of the C ABI's validation and planning layer (kda_abi.cpp, kda_plan.cpp) under
// AddressSanitizer and UndefinedBehaviorSanitizer. Both files are built for the host only; the
// kernel launchers and the three HIP runtime queries they use are replaced here by stubs that
// record what would have been enqueued. Built and run by tests/test_host_sanitizers.py: no GPU,
// no device memory; every data pointer is a fake address that nothing dereferences.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kda.h"
#include "kda_internal.h"
#include "kda_plan.h"

namespace {
int g_intra, g_inter, g_scan, g_chunk, g_copy, g_prep, g_bwd, g_decode, g_fused, g_lanes;
kda::ChunkLaunch g_last;
kda::ChunkLaunch g_inter_seq[8];   // the first state-pass launches since reset(), in order
kda::IntraArgs g_intra_seq[4];     // the first intra-chunk launches since reset()
kda::ChunkLaunch g_fused_last;
int g_order[16], g_norder;          // launch kinds in order: 1 intra, 2 inter, 3 scan, 4 fused, 5 lane list,
                                    // 6 window slot list
kda::WindowSlots g_wslots;
void note(int kind) { if (g_norder < 16) g_order[g_norder++] = kind; }
void reset() { g_intra = g_inter = g_scan = g_chunk = g_copy = g_prep = g_bwd = g_decode = g_fused = g_lanes = g_norder = 0; }
}  // namespace

namespace kda {
hipError_t launch_decode(const DecodeArgs& a, hipStream_t) { ++g_decode; return a.S && a.o ? hipSuccess : hipErrorInvalidValue; }
hipError_t launch_chunk(const ChunkLaunch& a, hipStream_t) { ++g_chunk; g_last = a; return hipSuccess; }
hipError_t launch_intra(const IntraArgs& a, hipStream_t) {
    if (g_intra < 4) g_intra_seq[g_intra] = a;
    ++g_intra; note(1);
    return a.rec ? hipSuccess : hipErrorInvalidValue;
}
hipError_t launch_inter(const ChunkLaunch& a, hipStream_t) {
    if (g_inter < 8) g_inter_seq[g_inter] = a;
    ++g_inter; g_last = a; note(2);
    return hipSuccess;
}
hipError_t launch_segment_scan(const ChunkLaunch&, hipStream_t) { ++g_scan; note(3); return hipSuccess; }
hipError_t launch_fused(const ChunkLaunch& a, hipStream_t) { ++g_fused; g_fused_last = a; note(4); return hipSuccess; }
hipError_t launch_fallback_lanes(const int32_t* flag, int64_t lanes, int nseg, int32_t* list, int32_t* count, hipStream_t) {
    ++g_lanes; note(5);
    return flag && list && count && lanes > 0 && nseg > 1 ? hipSuccess : hipErrorInvalidValue;
}
hipError_t launch_varlen_prep(const VarlenPrep&, hipStream_t) { ++g_prep; return hipSuccess; }
hipError_t launch_window_slots(const WindowSlots& a, hipStream_t) {
    g_wslots = a; note(6);
    return a.cu && a.list && a.count && a.nseg > 1 ? hipSuccess : hipErrorInvalidValue;
}
hipError_t launch_copy_or_zero(float* dst, const float*, int64_t n, hipStream_t) { ++g_copy; return dst && n > 0 ? hipSuccess : hipErrorInvalidValue; }
hipError_t launch_bwd(const BwdArgs& a, hipStream_t) { ++g_bwd; return a.ckpt || a.T < 64 ? hipSuccess : hipErrorInvalidValue; }
size_t bwd_prep_floats(int64_t dk, int64_t dv) { return (size_t)(64 * (3 * dk + dv) + 64 * 64 + dk); }
}  // namespace kda

extern "C" {
hipError_t hipGetDevice(int* d) { *d = 0; return hipSuccess; }
hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t* d) { *d = 0; return hipSuccess; }
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) { *v = 256; return hipSuccess; }
}

#define CHECK(cond)                                                               \
    do {                                                                          \
        if (!(cond)) {                                                            \
            fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);       \
            return 1;                                                             \
        }                                                                         \
    } while (0)

static const uintptr_t FAKE = 0x7F0000000000ull;
static void* P(uintptr_t off) { return reinterpret_cast<void*>(FAKE + off); }
static const uintptr_t GB = 1ull << 30;

static kda_chunk_desc cdesc(int64_t B, int64_t H, int64_t T, int64_t dk = 128, int64_t dv = 128, int32_t ind = KDA_BF16,
                            int32_t seg = 0) {
    kda_chunk_desc d;
    memset(&d, 0, sizeof(d));
    d.B = B; d.H = H; d.T = T; d.dk = dk; d.dv = dv; d.chunk = 64; d.in_dtype = ind; d.out_dtype = KDA_BF16; d.segments = seg;
    return d;
}

static kda_status fwd(const kda_chunk_desc* d, void* ws, size_t wsb, void* S0 = nullptr, void* ST = nullptr,
                      void* o = P(5 * GB), void* q = P(0)) {
    return kda_chunk_fwd(d, q, P(1 * GB), P(2 * GB), P(3 * GB), P(4 * GB), (const float*)S0, o, (float*)ST, ws, wsb, nullptr);
}

static void* scratch_stub(int) { return P(40 * GB); }

static int check_status_strings() {
    for (int s = 0; s >= -5; --s) CHECK(strncmp(kda_status_string(s), "KDA_", 4) == 0);
    CHECK(strcmp(kda_status_string(1234), "unknown kda_status") == 0);
    CHECK(strncmp(kda_version(), "kda-gfx950", 10) == 0);
    return 0;
}

static int check_chunk() {
    kda_chunk_desc d = cdesc(1, 2, 128);
    CHECK(kda_chunk_fwd_workspace_bytes(nullptr) == 0);
    CHECK(fwd(nullptr, nullptr, 0) == KDA_ERR_INVALID_ARG);
    kda_chunk_desc bad = d; bad.B = 0; CHECK(fwd(&bad, nullptr, 0) == KDA_ERR_INVALID_ARG);
    bad = d; bad.T = -1; CHECK(fwd(&bad, nullptr, 0) == KDA_ERR_INVALID_ARG);
    bad = d; bad.chunk = 32; CHECK(fwd(&bad, nullptr, 0) == KDA_ERR_UNSUPPORTED);
    bad = d; bad.dk = 96; CHECK(fwd(&bad, nullptr, 0) == KDA_ERR_UNSUPPORTED);
    bad = d; bad.in_dtype = 9; CHECK(fwd(&bad, nullptr, 0) == KDA_ERR_INVALID_ARG);
    bad = cdesc(1, 1, (int64_t)1 << 23); CHECK(fwd(&bad, nullptr, 0) == KDA_ERR_UNSUPPORTED);   // 32-bit row offsets
    const size_t need = kda_chunk_fwd_workspace_bytes(&d);
    CHECK(need > 0);
    reset();
    CHECK(fwd(&d, nullptr, 0) == KDA_ERR_WORKSPACE);
    CHECK(fwd(&d, P(7 * GB), need - 1) == KDA_ERR_WORKSPACE);
    CHECK(fwd(&d, P(7 * GB + 8), need) == KDA_ERR_INVALID_ARG);        // misaligned workspace
    CHECK(fwd(&d, P(64), need) == KDA_ERR_INVALID_ARG);                // workspace overlaps q
    CHECK(fwd(&d, P(7 * GB), need, nullptr, P(256)) == KDA_ERR_INVALID_ARG);          // S_T inside q
    CHECK(fwd(&d, P(7 * GB), need, P(6 * GB), P(6 * GB + 1024)) == KDA_ERR_INVALID_ARG);  // partial S0 / S_T overlap
    CHECK(fwd(&d, P(7 * GB), need, nullptr, nullptr, P(64)) == KDA_ERR_INVALID_ARG);  // o overlaps q
    CHECK(fwd(&d, P(7 * GB), need, nullptr, nullptr, P(5 * GB), P(8)) == KDA_ERR_INVALID_ARG);  // misaligned q
    CHECK(g_intra == 0 && g_inter == 0);                                // nothing enqueued on an error
    // valid calls: one pass, a forced split (intra, pass 1, scan, pass 2), in-place state, T = 0, fp32
    CHECK(fwd(&d, P(7 * GB), need, P(6 * GB), P(6 * GB)) == KDA_OK);
    CHECK(g_intra == 1 && g_inter >= 1);
    kda_chunk_desc s4 = cdesc(1, 2, 64 * 40, 128, 128, KDA_BF16, 4);
    const size_t need4 = kda_chunk_fwd_workspace_bytes(&s4);
    reset();
    CHECK(fwd(&s4, P(7 * GB), need4, nullptr, P(6 * GB)) == KDA_OK);
    // FINISH of all 4 segments (windows of 8 chunks before segments 1..3), then the fallback:
    // summaries of segments 1..2, the scan, FINISH of segments 1..3 whose window was inexact;
    // the flags are the workspace's last 2 x 4 int32
    CHECK(g_intra == 1 && g_inter == 3 && g_scan == 1);
    const kda::ChunkLaunch& w0 = g_inter_seq[0];
    const kda::ChunkLaunch& w1 = g_inter_seq[1];
    const kda::ChunkLaunch& w2 = g_inter_seq[2];
    CHECK(w0.split == kda::kPassWindowFinish && w0.fin_seg_lo == 0 && w0.fin_nseg == 4 && w0.sum_nseg == 0 &&
          w0.win_chunks == 8);
    CHECK(w1.split == kda::kPassCarry && w1.fin_nseg == 0 && w1.sum_seg_lo == 1 && w1.sum_nseg == 2);
    CHECK(w2.split == kda::kPassFinish && w2.fin_seg_lo == 1 && w2.fin_nseg == 3 && w2.sum_nseg == 0 && w2.nseg == 4);
    CHECK(w0.ws_flag == (int32_t*)((char*)P(7 * GB) + need4 - 2 * 4 * sizeof(int32_t)) && w2.ws_flag == w0.ws_flag);
    CHECK((char*)w0.ws_entry + 2 * 4 * 128 * 128 * sizeof(float) == (char*)w0.ws_flag);
    CHECK(w0.skip_flag == nullptr && w2.skip_flag == nullptr);
    // the fused plan, forced: the windows' records and the window launch, the fused kernel, the
    // fallback lane list and those lanes' records, then the window split above for those lanes.
    // Its workspace adds the window launch's flags and the lane list (2 lanes + count, 16 bytes).
    kda_chunk_desc s5 = s4;
    s5.state_pass = 2;
    const size_t need5 = kda_chunk_fwd_workspace_bytes(&s5);
    CHECK(need5 == need4 + 2 * 4 * sizeof(int32_t) + 16);
    reset();
    CHECK(fwd(&s5, P(7 * GB), need5 - 1, nullptr, P(6 * GB)) == KDA_ERR_WORKSPACE);
    CHECK(fwd(&s5, P(7 * GB), need5, nullptr, P(6 * GB)) == KDA_OK);
    const int order[9] = {1, 2, 4, 5, 1, 2, 2, 3, 2};
    CHECK(g_norder == 9 && memcmp(g_order, order, sizeof(order)) == 0);
    const int32_t* pre = (const int32_t*)((char*)P(7 * GB) + need4);
    CHECK(g_intra_seq[0].win_chunks == 8 && g_intra_seq[0].chunks_per_seg == 10 && g_intra_seq[0].nseg == 4 &&
          !g_intra_seq[0].lane_list);
    CHECK(g_intra_seq[1].win_chunks == 0 && g_intra_seq[1].lane_list == pre + 2 * 4 &&
          g_intra_seq[1].lane_count == g_intra_seq[1].lane_list + 2);
    const kda::ChunkLaunch& v0 = g_inter_seq[0];
    CHECK(v0.split == kda::kPassWindow && v0.fin_seg_lo == 1 && v0.fin_nseg == 3 && v0.sum_nseg == 0 && v0.ws_flag == pre &&
          v0.skip_flag == nullptr && v0.win_chunks == 8);
    CHECK(g_fused_last.ws_flag == pre && g_fused_last.nseg == 4 && g_fused_last.chunks_per_seg == 10 &&
          g_fused_last.ws_entry == v0.ws_entry && g_fused_last.S_T == P(6 * GB));
    CHECK(g_inter_seq[1].split == kda::kPassWindowFinish && g_inter_seq[1].skip_flag == pre &&
          g_inter_seq[1].ws_flag == pre - 2 * 4);
    CHECK(g_inter_seq[2].split == kda::kPassCarry && g_inter_seq[2].skip_flag == pre);
    CHECK(g_inter_seq[3].split == kda::kPassFinish && g_inter_seq[3].skip_flag == pre);
    // forced with one segment: the fused kernel alone
    kda_chunk_desc s1 = cdesc(1, 2, 64 * 40, 128, 128, KDA_BF16, 1);
    s1.state_pass = 2;
    reset();
    CHECK(fwd(&s1, P(7 * GB), kda_chunk_fwd_workspace_bytes(&s1), nullptr, P(6 * GB)) == KDA_OK);
    CHECK(g_fused == 1 && g_intra == 0 && g_inter == 0 && g_fused_last.nseg == 1);
    // forced two kernels; the fused kernel takes dk = dv = 128 only; state_pass outside 0..2
    kda_chunk_desc s2 = s4;
    s2.state_pass = 1;
    CHECK(kda_chunk_fwd_workspace_bytes(&s2) == need4);
    kda_chunk_desc s6 = cdesc(1, 2, 128, 64, 128);
    s6.state_pass = 2;
    CHECK(fwd(&s6, P(7 * GB), GB) == KDA_ERR_UNSUPPORTED);
    bad = d; bad.state_pass = 3; CHECK(fwd(&bad, nullptr, 0) == KDA_ERR_INVALID_ARG);
    bad = d; bad.state_pass = -1; CHECK(fwd(&bad, nullptr, 0) == KDA_ERR_INVALID_ARG);
    // the library's choice: the fused plan for 32 heads x 1M tokens (8 segments per lane, one
    // workgroup per compute unit) and 4 x 32 lanes x 64K tokens (2 segments), two kernels for 32
    // heads x 8K tokens
    kda::Geometry g1m{32, 16384, 32 * 16384, 128, 128, KDA_BF16, 0, 0, 32, 256};
    g1m.fused_ok = true;
    const kda::Plan p1m = kda::make_plan(g1m);
    CHECK(p1m.fused && p1m.nseg == 8 && p1m.chunks_per_seg == 2048);
    kda::Geometry g64k{128, 1024, 128 * 1024, 128, 128, KDA_BF16, 0, 0, 128, 256};   // B = 4, H = 32, T = 65536
    g64k.fused_ok = true;
    const kda::Plan p64k = kda::make_plan(g64k);
    CHECK(p64k.fused && p64k.nseg == 2);
    kda::Geometry g8k{32, 128, 32 * 128, 128, 128, KDA_BF16, 0, 0, 32, 256};
    g8k.fused_ok = true;
    CHECK(!kda::make_plan(g8k).fused);
    g1m.fused_ok = false;
    CHECK(!kda::make_plan(g1m).fused);
    kda_chunk_desc z = cdesc(1, 2, 0);
    reset();
    CHECK(fwd(&z, nullptr, 0, nullptr, P(6 * GB)) == KDA_OK && g_copy == 1);
    kda_chunk_desc f = cdesc(1, 1, 256, 64, 64, KDA_F32);
    CHECK(kda_chunk_fwd_workspace_bytes(&f) == 0);
    reset();
    CHECK(fwd(&f, nullptr, 0) == KDA_OK && g_chunk == 1 && g_intra == 0);
    // the no-allocation variant: scratch looked up only after validation, too-large calls refused
    reset();
    CHECK(kda::chunk_fwd_impl(&d, P(0), P(GB), P(2 * GB), P(3 * GB), P(4 * GB), nullptr, P(5 * GB), nullptr, nullptr, 0,
                              nullptr, scratch_stub) == KDA_OK);
    kda_chunk_desc big = cdesc(1, 32, 8192);
    CHECK(kda::chunk_fwd_impl(&big, P(0), P(GB), P(2 * GB), P(3 * GB), P(4 * GB), nullptr, P(5 * GB), nullptr, nullptr, 0,
                              nullptr, scratch_stub) == KDA_ERR_SCRATCH);
    CHECK(kda::chunk_fwd_impl(&d, nullptr, P(GB), P(2 * GB), P(3 * GB), P(4 * GB), nullptr, P(5 * GB), nullptr, nullptr,
                              0, nullptr, scratch_stub) == KDA_ERR_INVALID_ARG);
    return 0;
}

static int check_varlen() {
    kda_varlen_desc d;
    memset(&d, 0, sizeof(d));
    d.N = 3; d.H = 2; d.T = 640; d.max_len = 512; d.dk = 128; d.dv = 128; d.chunk = 64; d.in_dtype = KDA_BF16;
    d.out_dtype = KDA_BF16; d.ckpt_every = 128; d.packed = 1;
    const size_t need = kda_chunk_fwd_varlen_workspace_bytes(&d);
    CHECK(need > 0);
    auto call = [&](const kda_varlen_desc* dd, void* cu, void* ck, void* cko, const kda_gating* g, void* ws, size_t wsb,
                    void* la = P(3 * GB)) {
        return kda_chunk_fwd_varlen(dd, P(0), P(GB), P(2 * GB), la, P(4 * GB), (const int32_t*)cu, nullptr, P(5 * GB),
                                    (float*)P(6 * GB), (float*)ck, (int32_t*)cko, g, ws, wsb, nullptr);
    };
    reset();
    CHECK(call(&d, P(8 * GB), P(9 * GB), P(10 * GB), nullptr, P(11 * GB), need) == KDA_OK);
    CHECK(g_prep == 1 && g_intra == 1 && g_inter >= 1);
    CHECK(call(&d, nullptr, P(9 * GB), P(10 * GB), nullptr, P(11 * GB), need) == KDA_ERR_INVALID_ARG);   // packed needs cu
    CHECK(call(&d, P(8 * GB), P(9 * GB), nullptr, nullptr, P(11 * GB), need) == KDA_ERR_INVALID_ARG);   // needs offsets
    CHECK(call(&d, P(8 * GB), P(9 * GB), P(9 * GB + 64), nullptr, P(11 * GB), need) == KDA_ERR_INVALID_ARG);  // overlap
    CHECK(call(&d, P(8 * GB), P(9 * GB), P(10 * GB), nullptr, P(11 * GB), need - 1) == KDA_ERR_WORKSPACE);
    kda_varlen_desc e = d; e.ckpt_every = 100; CHECK(call(&e, P(8 * GB), P(9 * GB), P(10 * GB), nullptr, P(11 * GB), need) == KDA_ERR_INVALID_ARG);
    kda_gating g;
    memset(&g, 0, sizeof(g));
    g.z = P(12 * GB); g.A_log = (const float*)P(13 * GB); g.g_min = -5.f; g.gate = P(14 * GB); g.eps = 1e-6f;
    reset();
    CHECK(call(&d, P(8 * GB), P(9 * GB), P(10 * GB), &g, P(11 * GB), need, nullptr) == KDA_OK && g_intra == 1);
    g.g_min = 0.f;
    CHECK(call(&d, P(8 * GB), P(9 * GB), P(10 * GB), &g, P(11 * GB), need, nullptr) == KDA_ERR_INVALID_ARG);
    g.g_min = -5.f;
    // the plan of a packed batch splits for the lanes that can be long: 12 sequences x 32 heads,
    // 8192 tokens, longest 2500 (40 chunks; at most 3 sequences that long): 2 segments
    {
        kda_varlen_desc pk = d;
        pk.N = 12; pk.H = 32; pk.T = 8192; pk.max_len = 2500; pk.ckpt_every = 512;
        const size_t needk = kda_chunk_fwd_varlen_workspace_bytes(&pk);
        reset();
        CHECK(call(&pk, P(8 * GB), P(9 * GB), P(10 * GB), nullptr, P(11 * GB), needk) == KDA_OK);
        CHECK(g_fused == 0 && g_inter >= 1 && g_inter_seq[0].nseg == 2 && g_inter_seq[0].chunks_per_seg == 20);
    }
    // the fused kernel on a packed batch (3 segments of 4 chunks): the slot table, the list of the
    // windows' slots and their records, the window launch, the fused kernel, the lane list, every
    // record when a lane falls back, then the two-kernel passes skipping the fused lanes
    kda_varlen_desc f = d;
    f.state_pass = 2; f.segments = 3; f.max_len = 768; f.T = 1536;
    const size_t needp = kda_chunk_fwd_varlen_workspace_bytes(&f);
    kda_varlen_desc f1 = f; f1.state_pass = 1;
    CHECK(needp > kda_chunk_fwd_varlen_workspace_bytes(&f1));
    reset();
    CHECK(call(&f, P(8 * GB), P(9 * GB), P(10 * GB), nullptr, P(11 * GB), needp - 1) == KDA_ERR_WORKSPACE);
    CHECK(call(&f, P(8 * GB), P(9 * GB), P(10 * GB), nullptr, P(11 * GB), needp) == KDA_OK);
    {
        const int want[] = {6, 1, 2, 4, 5, 1, 2, 2, 3, 2};
        CHECK(g_norder == 10 && g_prep == 1);
        for (int i = 0; i < 10; ++i) CHECK(g_order[i] == want[i]);
        const unsigned char* w0 = (const unsigned char*)P(11 * GB);
        const unsigned char* wend = w0 + needp;
        CHECK(g_wslots.N == 3 && g_wslots.H == 2 && g_wslots.nseg == 3 && g_wslots.chunks_per_seg == 4 &&
              g_wslots.win_chunks == 8 && g_wslots.max_len == 768 && g_wslots.rows == 1536);
        CHECK((const unsigned char*)g_wslots.list > w0 && (const unsigned char*)(g_wslots.count + 1) <= wend &&
              g_wslots.count == g_wslots.list + 6 * 2 * 8);
        CHECK(g_intra_seq[0].slot_list == g_wslots.list && g_intra_seq[0].slot_count == g_wslots.count &&
              g_intra_seq[0].slot_tab != nullptr && g_intra_seq[0].run_if == nullptr);
        CHECK(g_intra_seq[1].slot_list == nullptr && g_intra_seq[1].lane_list == nullptr && g_intra_seq[1].run_if &&
              (const unsigned char*)g_intra_seq[1].run_if < (const unsigned char*)g_wslots.list);
        CHECK(g_inter_seq[0].split == kda::kPassWindow && g_inter_seq[0].map.cu == P(8 * GB));
        CHECK(g_fused_last.map.cu == P(8 * GB) && g_fused_last.ws_flag == g_inter_seq[0].ws_flag && g_fused_last.nseg == 3);
        for (int i = 1; i < 4; ++i) CHECK(g_inter_seq[i].skip_flag == g_inter_seq[0].ws_flag);
    }
    f.packed = 0; f.segments = 2; f.max_len = 512; f.T = 640;
    const size_t needf = kda_chunk_fwd_varlen_workspace_bytes(&f);
    reset();
    CHECK(call(&f, nullptr, P(9 * GB), P(10 * GB), &g, P(11 * GB), needf, nullptr) == KDA_OK);
    CHECK(g_fused == 1 && g_fused_last.ckpt == (float*)P(9 * GB) && g_fused_last.ck_chunks == 2 &&
          g_fused_last.gt.z == P(12 * GB) && g_fused_last.gt.gate == P(14 * GB) && g_fused_last.nseg == 2);
    f.state_pass = 3;
    CHECK(call(&f, nullptr, P(9 * GB), P(10 * GB), &g, P(11 * GB), needf, nullptr) == KDA_ERR_INVALID_ARG);
    return 0;
}

static int check_bwd_and_decode() {
    kda_chunk_desc d = cdesc(1, 2, 256);
    const size_t need = kda_chunk_bwd_workspace_bytes(&d);
    CHECK(need > kda_chunk_fwd_workspace_bytes(&d));
    auto bwd = [&](void* q, void* ws, size_t wsb) {
        return kda_chunk_bwd(&d, q, P(GB), P(2 * GB), P(3 * GB), P(4 * GB), nullptr, P(5 * GB), nullptr, (float*)P(6 * GB),
                             (float*)P(7 * GB), (float*)P(8 * GB), (float*)P(9 * GB), (float*)P(10 * GB),
                             (float*)P(11 * GB), ws, wsb, nullptr);
    };
    reset();
    CHECK(bwd(P(0), P(12 * GB), need) == KDA_OK && g_bwd == 1 && g_intra == 1);
    CHECK(bwd(P(4), P(12 * GB), need) == KDA_ERR_INVALID_ARG);          // 16-byte alignment of q
    CHECK(bwd(P(0), P(12 * GB + 16), need) == KDA_ERR_INVALID_ARG);     // 256-byte workspace alignment
    CHECK(bwd(P(0), P(12 * GB), need - 1) == KDA_ERR_WORKSPACE);
    d.state_pass = 1;
    CHECK(kda_chunk_bwd_workspace_bytes(&d) == need && bwd(P(0), P(12 * GB), need) == KDA_OK);
    d.state_pass = 2;   // the backward's forward keeps its checkpoints: two kernels only
    CHECK(bwd(P(0), P(12 * GB), need) == KDA_ERR_UNSUPPORTED);
    d.state_pass = 0;
    kda_decode_desc dd;
    memset(&dd, 0, sizeof(dd));
    dd.N = 4; dd.H = 2; dd.dk = 128; dd.dv = 128; dd.in_dtype = KDA_BF16; dd.out_dtype = KDA_BF16;
    reset();
    CHECK(kda_decode_step(&dd, P(0), P(GB), P(2 * GB), P(3 * GB), P(4 * GB), (float*)P(5 * GB), P(6 * GB), nullptr) == KDA_OK);
    CHECK(g_decode == 1);
    CHECK(kda_decode_step(&dd, P(0), P(GB), P(2 * GB), P(3 * GB), P(4 * GB), (float*)P(5 * GB), P(5 * GB + 64), nullptr) ==
          KDA_ERR_INVALID_ARG);                                          // o overlaps S
    dd.dk = 80;
    CHECK(kda_decode_step(&dd, P(0), P(GB), P(2 * GB), P(3 * GB), P(4 * GB), (float*)P(5 * GB), P(6 * GB), nullptr) ==
          KDA_ERR_UNSUPPORTED);
    return 0;
}

int main() {
    if (check_status_strings() || check_chunk() || check_varlen() || check_bwd_and_decode()) return 1;
    printf("abi host check: ok\n");
    return 0;
}
