// Host-layer checks of libdsaidx under AddressSanitizer and
// UndefinedBehaviorSanitizer, on the CPU.  dsaidx_api.cpp is linked against
// stubs of the kernel launchers and of the two HIP device queries, which
// record what the host layer asks for.  Pointers are real, aligned host
// memory that nothing dereferences.  Exit status 0 when every check passes.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "dsaidx.h"
#include "dsaidx_internal.h"

namespace {

struct Launch {
    int kind;  // 0 prep, 1 top-k, 2 fp8 self-test, 3 logits, 4 HBM stream, 5 projection
    dsaidx::PrepParams p;
    dsaidx::LogitsParams lp;
    int style;
    unsigned grid, block;
    int64_t rows, cols, row_stride, n;
    int32_t k;
    const void* workspace;
};

std::vector<Launch> g_launches;
hipError_t g_fail = hipSuccess;  // what the launch stubs return
int g_errors = 0;

#define CHECK(c)                                                                   \
    do {                                                                           \
        if (!(c)) {                                                                \
            std::fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #c);    \
            ++g_errors;                                                            \
        }                                                                          \
    } while (0)

alignas(64) unsigned char g_arena[1 << 16];

template <typename P>
P* at(size_t off) { return reinterpret_cast<P*>(g_arena + off); }

}  // namespace

namespace dsaidx {

hipError_t launch_prep(const PrepParams& p, int style, unsigned grid, unsigned block, hipStream_t) {
    Launch l;
    std::memset(&l, 0, sizeof l);
    l.kind = 0;
    l.p = p;
    l.style = style;
    l.grid = grid;
    l.block = block;
    g_launches.push_back(l);
    return g_fail;
}

hipError_t launch_topk(const float*, int64_t row_stride, const int32_t*, int64_t rows, int64_t cols,
                       int32_t k, int32_t*, void* workspace, hipStream_t) {
    Launch l;
    std::memset(&l, 0, sizeof l);
    l.kind = 1;
    l.rows = rows;
    l.cols = cols;
    l.row_stride = row_stride;
    l.k = k;
    l.workspace = workspace;
    g_launches.push_back(l);
    return g_fail;
}

hipError_t launch_fp8_selftest(const float*, uint8_t*, int64_t n, float scale, unsigned grid, hipStream_t) {
    CHECK(scale > 0.0f);
    Launch l;
    std::memset(&l, 0, sizeof l);
    l.kind = 2;
    l.n = n;
    l.grid = grid;
    g_launches.push_back(l);
    return g_fail;
}

hipError_t launch_logits(const LogitsParams& p, hipStream_t) {
    Launch l;
    std::memset(&l, 0, sizeof l);
    l.kind = 3;
    l.lp = p;
    g_launches.push_back(l);
    return g_fail;
}

hipError_t launch_proj(const ProjParams& p, int style, unsigned grid, hipStream_t) {
    Launch l;
    std::memset(&l, 0, sizeof l);
    l.kind = 5;
    l.p = p.prep;
    l.style = style;
    l.grid = grid;
    l.n = p.d;
    l.rows = p.row_blocks;
    l.k = p.H;
    l.row_stride = p.x_st;
    l.workspace = p.k_out;
    g_launches.push_back(l);
    return g_fail;
}

hipError_t launch_hbm_stream(int mode, const void*, void*, int64_t vectors, uint32_t, hipStream_t) {
    Launch l;
    std::memset(&l, 0, sizeof l);
    l.kind = 4;
    l.n = vectors;
    l.style = mode;
    g_launches.push_back(l);
    return g_fail;
}

int g_scratch_lookups = 0;
hipError_t topk_scratch(int, void** ptr) {
    ++g_scratch_lookups;
    *ptr = reinterpret_cast<void*>(uintptr_t(1) << 40);
    return hipSuccess;
}

// The size include/dsaidx.h documents.
int64_t topk_workspace_bytes(int64_t rows, int64_t cols, int32_t) {
    if (cols <= 32768) return 0;
    if (rows * ((cols + 4095) / 4096) >= (int64_t(1) << 31)) return -1;
    int64_t list = cols / 16 > 4096 ? cols / 16 : 4096;
    list = (list + 3) / 4 * 4;
    return rows * (8224 + 8 * list);
}

}  // namespace dsaidx

extern "C" {
hipError_t hipGetDeviceCount(int* count) {
    *count = 0;
    return hipErrorNoDevice;
}
hipError_t hipGetDeviceProperties(hipDeviceProp_t*, int) { return hipErrorNoDevice; }
int g_current_device = 0;
int g_stream_device = 0;
hipError_t hipGetDevice(int* device) {
    *device = g_current_device;
    return hipSuccess;
}
hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t* device) {
    *device = g_stream_device;
    return hipSuccess;
}
}

namespace {

dsaidx_rope make_rope() {
    dsaidx_rope r;
    std::memset(&r, 0, sizeof r);
    r.cos = at<const float>(0);
    r.sin = at<const float>(1024);
    r.row_stride = 32;
    r.max_position = 4096;
    r.rope_dim = 64;
    r.style = DSAIDX_ROPE_NEOX;
    return r;
}

dsaidx_q_args make_q(int64_t T, int32_t H) {
    dsaidx_q_args q;
    std::memset(&q, 0, sizeof q);
    q.q = at<const uint16_t>(2048);
    q.q_stride_h = 128;
    q.q_stride_t = 128 * (int64_t)H;
    q.weights = at<const uint16_t>(4096);
    q.w_stride_t = H;
    q.positions = at<const int64_t>(6144);
    q.num_tokens = T;
    q.num_heads = H;
    q.weight_scale = 1.0f;
    q.q_fp8 = at<uint8_t>(8192);
    q.weights_out = at<float>(10240);
    q.q_scale_out = nullptr;
    return q;
}

dsaidx_k_args make_k(int64_t T) {
    dsaidx_k_args k;
    std::memset(&k, 0, sizeof k);
    k.k = at<const uint16_t>(12288);
    k.k_stride_t = 128;
    k.ln_gamma = at<const float>(14336);
    k.ln_beta = at<const float>(16384);
    k.ln_eps = 1e-6f;
    k.flags = 0;
    k.positions = at<const int64_t>(18432);
    k.out_cache_loc = at<const int64_t>(20480);
    k.num_tokens = T;
    k.k_cache = at<uint8_t>(22528);
    k.k_cache_row_stride = 128;
    k.k_scale = at<float>(24576);
    k.num_slots = 4096;
    k.page_size = 0;
    return k;
}

// Runs f (which must return DSAIDX_ERR_INVALID_ARGUMENT) and checks that it
// enqueued nothing.
template <typename F>
void expect_rejected(F f, int line) {
    const size_t before = g_launches.size();
    const dsaidx_status st = f();
    if (st != DSAIDX_ERR_INVALID_ARGUMENT || g_launches.size() != before) {
        std::fprintf(stderr, "FAILED line %d: status %d, launches %zu -> %zu\n", line, (int)st, before,
                     g_launches.size());
        ++g_errors;
    }
}
#define REJECT(expr) expect_rejected([&] { return (expr); }, __LINE__)

void abi_and_status() {
    CHECK(dsaidx_abi_version() == DSAIDX_ABI_VERSION);
    const dsaidx_status all[] = {DSAIDX_OK, DSAIDX_ERR_INVALID_ARGUMENT, DSAIDX_ERR_UNSUPPORTED,
                                 DSAIDX_ERR_HIP};
    for (dsaidx_status s : all) {
        const char* t = dsaidx_status_string(s);
        CHECK(t != nullptr && std::strlen(t) > 0);
    }
    CHECK(dsaidx_device_supported(0) == 0);
    CHECK(dsaidx_device_supported(-1) == 0);
}

void launch_shapes() {
    const dsaidx_rope rope = make_rope();
    // fused, small batch: 4-head items, T * H = 320 query rows
    {
        g_launches.clear();
        dsaidx_q_args q = make_q(5, 64);
        dsaidx_k_args k = make_k(5);
        CHECK(dsaidx_qk_fused(&q, &k, &rope, nullptr) == DSAIDX_OK);
        CHECK(g_launches.size() == 1);
        const Launch& l = g_launches[0];
        CHECK(l.kind == 0 && l.block == 256 && l.style == DSAIDX_ROPE_NEOX);
        CHECK(l.p.heads_per_item == 4 && l.p.head_blocks == 16 && l.p.q_items == 80);
        CHECK(l.p.k_items == 2 && l.p.k_blocks == 1 && l.grid == 20 + 1);
        CHECK(l.p.T == 5 && l.p.H == 64 && l.p.R == 64 && l.p.P == 4096 && l.p.rs == 32);
        CHECK(l.p.page_size == 0 && l.p.S == 4096 && l.p.eps == 1e-6f && l.p.q_scale == nullptr);
        CHECK(l.p.k_first == 0);                 // fewer than 32 tokens: key workgroups last
        CHECK(l.p.k_period == 0);
    }
    // fused, small batch of 64 tokens: key workgroups first, none capped
    {
        g_launches.clear();
        dsaidx_q_args q = make_q(64, 64);
        dsaidx_k_args k = make_k(64);
        CHECK(dsaidx_qk_fused(&q, &k, &rope, nullptr) == DSAIDX_OK);
        const Launch& l = g_launches[0];
        CHECK(l.p.heads_per_item == 4 && l.p.k_first == 1 && l.p.k_blocks == 4 && l.grid == 256 + 4);
    }
    // fused, large batch: 16-head items; key workgroups capped at 1/16 of the query ones
    {
        g_launches.clear();
        dsaidx_q_args q = make_q(300, 64);
        dsaidx_k_args k = make_k(300);
        CHECK(dsaidx_qk_fused(&q, &k, &rope, nullptr) == DSAIDX_OK);
        CHECK(g_launches.size() == 1);
        const Launch& l = g_launches[0];
        CHECK(l.p.heads_per_item == 16 && l.p.head_blocks == 4 && l.p.q_items == 1200);
        CHECK(l.p.k_items == 75 && l.p.k_blocks == 19 && l.grid == 300 + 19);
        CHECK(l.p.k_first == 0);
    }
    // fused, large batch of exactly 8 heads: items of two tokens x 8 heads, key
    // workgroups not capped
    {
        g_launches.clear();
        dsaidx_q_args q = make_q(4097, 8);
        dsaidx_k_args k = make_k(4097);
        CHECK(dsaidx_qk_fused(&q, &k, &rope, nullptr) == DSAIDX_OK);
        CHECK(g_launches.size() == 1);
        const Launch& l = g_launches[0];
        CHECK(l.p.heads_per_item == 8 && l.p.head_blocks == 1 && l.p.q_items == 2049);
        CHECK(l.p.k_items == 1025 && l.p.k_blocks == 257 && l.grid == 513 + 257);
        CHECK(l.p.k_period == 0);                // one resident round: key workgroups last
    }
    // fused 8-head calls of several rounds: key workgroups spread through the grid.
    // The kernel's split of the workgroup index (one key workgroup at the end
    // of each period, query workgroups past the last period) must give every
    // key and query workgroup index exactly once.
    for (const auto& shape : {std::pair<int64_t, int32_t>{65536, 8}, {30001, 8}, {20000, 8}}) {
        g_launches.clear();
        dsaidx_q_args q = make_q(shape.first, shape.second);
        dsaidx_k_args k = make_k(shape.first);
        CHECK(dsaidx_qk_fused(&q, &k, &rope, nullptr) == DSAIDX_OK);
        CHECK(g_launches.size() == 1);
        const Launch& l = g_launches[0];
        CHECK(l.p.k_period >= 2 && l.p.k_blocks > 0);
        if (l.p.k_period < 2 || l.p.k_blocks <= 0) continue;
        const uint32_t per = (uint32_t)l.p.k_period, kbn = (uint32_t)l.p.k_blocks;
        const uint32_t nq = l.grid - kbn;
        std::vector<int> seen_k(kbn, 0), seen_q(nq, 0);
        for (uint32_t b = 0; b < l.grid; ++b) {
            const uint32_t j = (uint32_t)(((uint64_t)b * l.p.k_magic) >> l.p.k_shift);
            CHECK(j == b / per);
            const uint32_t i = b - j * per;
            if (j < kbn && i == per - 1) {
                ++seen_k[j];
            } else {
                const uint64_t qb = j < kbn ? (uint64_t)j * (per - 1) + i : (uint64_t)kbn * (per - 1) + (b - kbn * per);
                CHECK(qb < nq);
                if (qb < nq) ++seen_q[qb];
            }
        }
        for (int c : seen_k) CHECK(c == 1);
        for (int c : seen_q) CHECK(c == 1);
    }
    // at 64 heads the key workgroups stay last whatever the size
    for (int64_t T : {8192, 65536}) {
        g_launches.clear();
        dsaidx_q_args q = make_q(T, 64);
        dsaidx_k_args k = make_k(T);
        CHECK(dsaidx_qk_fused(&q, &k, &rope, nullptr) == DSAIDX_OK);
        CHECK(g_launches.size() == 1 && g_launches[0].p.k_period == 0);
    }
    // query side alone, interleaved rope, odd head count
    {
        g_launches.clear();
        dsaidx_rope r2 = rope;
        r2.style = DSAIDX_ROPE_INTERLEAVED;
        dsaidx_q_args q = make_q(7, 5);
        q.q_scale_out = at<float>(26624);
        CHECK(dsaidx_q_rope_quant_fold(&q, &r2, nullptr) == DSAIDX_OK);
        CHECK(g_launches.size() == 1);
        const Launch& l = g_launches[0];
        CHECK(l.style == DSAIDX_ROPE_INTERLEAVED && l.p.k_blocks == 0 && l.p.k_items == 0);
        CHECK(l.p.head_blocks == 2 && l.p.q_items == 14 && l.grid == 4 && l.p.q_scale != nullptr);
    }
    // key side alone, and the k-only entry's one-wavefront workgroups
    {
        g_launches.clear();
        dsaidx_k_args k = make_k(9);
        CHECK(dsaidx_k_norm_rope_quant_store(&k, &rope, nullptr) == DSAIDX_OK);
        CHECK(dsaidx_k_only_prepare_store(&k, &rope, nullptr) == DSAIDX_OK);
        CHECK(g_launches.size() == 2);
        CHECK(g_launches[0].p.k_items == 3 && g_launches[0].grid == 1 && g_launches[0].block == 256);
        CHECK(g_launches[0].p.q_items == 0 && g_launches[0].p.k_blocks == 1);
        CHECK(g_launches[1].grid == 3 && g_launches[1].block == 64 && g_launches[1].p.k_blocks == 3);
    }
    // page-interleaved cache: no planar scale array needed
    {
        g_launches.clear();
        dsaidx_k_args k = make_k(4);
        k.flags = DSAIDX_K_PAGED_CACHE | DSAIDX_K_BF16_INTERMEDIATE;
        k.page_size = 64;
        k.k_scale = nullptr;
        k.k_cache_row_stride = 0;
        CHECK(dsaidx_k_norm_rope_quant_store(&k, &rope, nullptr) == DSAIDX_OK);
        CHECK(g_launches.size() == 1 && g_launches[0].p.page_size == 64);
        CHECK(g_launches[0].p.k_flags == (DSAIDX_K_PAGED_CACHE | DSAIDX_K_BF16_INTERMEDIATE));
        g_launches.clear();
        k.flags = DSAIDX_K_PAGED_CACHE | DSAIDX_K_BF16_ROUND_ONCE;
        CHECK(dsaidx_k_norm_rope_quant_store(&k, &rope, nullptr) == DSAIDX_OK);
        CHECK(g_launches.size() == 1 && g_launches[0].p.k_flags == (DSAIDX_K_PAGED_CACHE | DSAIDX_K_BF16_ROUND_ONCE));
    }
    // no tokens: nothing enqueued, from any entry
    {
        g_launches.clear();
        dsaidx_q_args q = make_q(0, 64);
        dsaidx_k_args k = make_k(0);
        q.q = nullptr;  // not looked at when there is nothing to do
        CHECK(dsaidx_qk_fused(&q, &k, &rope, nullptr) == DSAIDX_OK);
        CHECK(dsaidx_q_rope_quant_fold(&q, &rope, nullptr) == DSAIDX_OK);
        CHECK(dsaidx_k_norm_rope_quant_store(&k, &rope, nullptr) == DSAIDX_OK);
        CHECK(dsaidx_k_only_prepare_store(&k, &rope, nullptr) == DSAIDX_OK);
        CHECK(g_launches.empty());
    }
    // launch errors map to status codes
    {
        dsaidx_q_args q = make_q(3, 8);
        g_fail = hipErrorNoBinaryForGpu;
        CHECK(dsaidx_q_rope_quant_fold(&q, &rope, nullptr) == DSAIDX_ERR_UNSUPPORTED);
        g_fail = hipErrorOutOfMemory;
        CHECK(dsaidx_q_rope_quant_fold(&q, &rope, nullptr) == DSAIDX_ERR_HIP);
        g_fail = hipSuccess;
    }
}

void rejected_arguments() {
    const dsaidx_rope rope = make_rope();
    const dsaidx_q_args q0 = make_q(3, 8);
    const dsaidx_k_args k0 = make_k(3);
    g_launches.clear();
    REJECT(dsaidx_q_rope_quant_fold(nullptr, &rope, nullptr));
    REJECT(dsaidx_q_rope_quant_fold(&q0, nullptr, nullptr));
    REJECT(dsaidx_qk_fused(&q0, nullptr, &rope, nullptr));
    {
        dsaidx_k_args k = k0;
        k.num_tokens = 4;  // the two sides must agree
        REJECT(dsaidx_qk_fused(&q0, &k, &rope, nullptr));
    }
    // rope table
    auto bad_rope = [&](void (*edit)(dsaidx_rope&)) {
        dsaidx_rope r = rope;
        edit(r);
        dsaidx_q_args q = q0;
        dsaidx_k_args k = k0;
        REJECT(dsaidx_q_rope_quant_fold(&q, &r, nullptr));
        REJECT(dsaidx_k_norm_rope_quant_store(&k, &r, nullptr));
        REJECT(dsaidx_qk_fused(&q, &k, &r, nullptr));
    };
    // rope_dim not a multiple of 16, a row stride not a multiple of 4 or rows
    // not 16-byte aligned: the element-wise path, never two-token items
    {
        auto path = [&](void (*edit)(dsaidx_rope&), int64_t T, int32_t H) {
            dsaidx_rope r = rope;
            edit(r);
            dsaidx_q_args q = make_q(T, H);
            dsaidx_k_args k = make_k(T);
            g_launches.clear();
            CHECK(dsaidx_qk_fused(&q, &k, &r, nullptr) == DSAIDX_OK);
            CHECK(g_launches.size() == 1);
            return g_launches.empty() ? Launch{} : g_launches[0];
        };
        CHECK(path([](dsaidx_rope&) {}, 64, 64).p.generic == 0);
        CHECK(path([](dsaidx_rope& r) { r.rope_dim = 24; }, 64, 64).p.generic == 1);
        CHECK(path([](dsaidx_rope& r) { r.rope_dim = 2; r.row_stride = 1; }, 64, 64).p.generic == 1);
        CHECK(path([](dsaidx_rope& r) { r.row_stride = 33; }, 64, 64).p.generic == 1);
        CHECK(path([](dsaidx_rope& r) { r.sin = at<const float>(1028); }, 64, 64).p.generic == 1);
        const Launch fast8 = path([](dsaidx_rope&) {}, 65536, 8);
        CHECK(fast8.p.generic == 0 && fast8.p.heads_per_item == 8);
        const Launch slow8 = path([](dsaidx_rope& r) { r.row_stride = 33; }, 65536, 8);
        CHECK(slow8.p.generic == 1 && slow8.p.heads_per_item == 16 && slow8.p.q_items == 65536);
        g_launches.clear();
    }
    bad_rope([](dsaidx_rope& r) { r.cos = nullptr; });
    bad_rope([](dsaidx_rope& r) { r.sin = at<const float>(1026); });      // not 4-byte aligned
    bad_rope([](dsaidx_rope& r) { r.rope_dim = 0; });
    bad_rope([](dsaidx_rope& r) { r.rope_dim = 23; });                    // odd
    bad_rope([](dsaidx_rope& r) { r.rope_dim = 144; });
    bad_rope([](dsaidx_rope& r) { r.style = 2; });
    bad_rope([](dsaidx_rope& r) { r.row_stride = 16; });                  // < rope_dim / 2
    bad_rope([](dsaidx_rope& r) { r.rope_dim = 10; r.row_stride = 4; });  // < rope_dim / 2
    bad_rope([](dsaidx_rope& r) { r.max_position = 0; });
    // query side
    auto bad_q = [&](void (*edit)(dsaidx_q_args&)) {
        dsaidx_q_args q = q0;
        edit(q);
        dsaidx_k_args k = k0;
        k.num_tokens = q.num_tokens;
        REJECT(dsaidx_q_rope_quant_fold(&q, &rope, nullptr));
        REJECT(dsaidx_qk_fused(&q, &k, &rope, nullptr));
    };
    bad_q([](dsaidx_q_args& q) { q.num_tokens = -1; });
    bad_q([](dsaidx_q_args& q) { q.num_heads = 0; });
    bad_q([](dsaidx_q_args& q) { q.num_heads = 4097; });
    bad_q([](dsaidx_q_args& q) { q.weight_scale = INFINITY; });
    bad_q([](dsaidx_q_args& q) { q.weight_scale = NAN; });
    bad_q([](dsaidx_q_args& q) { q.q = nullptr; });
    bad_q([](dsaidx_q_args& q) { q.weights = nullptr; });
    bad_q([](dsaidx_q_args& q) { q.positions = nullptr; });
    bad_q([](dsaidx_q_args& q) { q.q_fp8 = nullptr; });
    bad_q([](dsaidx_q_args& q) { q.weights_out = nullptr; });
    bad_q([](dsaidx_q_args& q) { q.q = at<const uint16_t>(2056); });      // 8-byte aligned only
    bad_q([](dsaidx_q_args& q) { q.weights = at<const uint16_t>(4097); });
    bad_q([](dsaidx_q_args& q) { q.positions = at<const int64_t>(6148); });
    bad_q([](dsaidx_q_args& q) { q.q_fp8 = at<uint8_t>(8196); });
    bad_q([](dsaidx_q_args& q) { q.weights_out = at<float>(10242); });
    bad_q([](dsaidx_q_args& q) { q.q_scale_out = at<float>(26626); });
    bad_q([](dsaidx_q_args& q) { q.q_stride_h = 120; });
    bad_q([](dsaidx_q_args& q) { q.q_stride_h = 132; });                 // not a multiple of 8
    bad_q([](dsaidx_q_args& q) { q.q_stride_t = 7 * 128 + 120; });      // rows would overlap
    bad_q([](dsaidx_q_args& q) { q.q_stride_t = 8 * 128 + 4; });
    bad_q([](dsaidx_q_args& q) { q.w_stride_t = 7; });
    // key side
    auto bad_k = [&](void (*edit)(dsaidx_k_args&)) {
        dsaidx_k_args k = k0;
        edit(k);
        dsaidx_q_args q = q0;
        q.num_tokens = k.num_tokens;
        REJECT(dsaidx_k_norm_rope_quant_store(&k, &rope, nullptr));
        REJECT(dsaidx_k_only_prepare_store(&k, &rope, nullptr));
        REJECT(dsaidx_qk_fused(&q, &k, &rope, nullptr));
    };
    bad_k([](dsaidx_k_args& k) { k.num_tokens = -5; });
    bad_k([](dsaidx_k_args& k) { k.k = nullptr; });
    bad_k([](dsaidx_k_args& k) { k.ln_gamma = nullptr; });
    bad_k([](dsaidx_k_args& k) { k.ln_beta = nullptr; });
    bad_k([](dsaidx_k_args& k) { k.positions = nullptr; });
    bad_k([](dsaidx_k_args& k) { k.out_cache_loc = nullptr; });
    bad_k([](dsaidx_k_args& k) { k.k_cache = nullptr; });
    bad_k([](dsaidx_k_args& k) { k.k_scale = nullptr; });
    bad_k([](dsaidx_k_args& k) { k.k = at<const uint16_t>(12296); });
    bad_k([](dsaidx_k_args& k) { k.ln_gamma = at<const float>(14340); });
    bad_k([](dsaidx_k_args& k) { k.out_cache_loc = at<const int64_t>(20484); });
    bad_k([](dsaidx_k_args& k) { k.k_scale = at<float>(24577); });
    bad_k([](dsaidx_k_args& k) { k.k_stride_t = 64; });
    bad_k([](dsaidx_k_args& k) { k.k_stride_t = 132; });
    bad_k([](dsaidx_k_args& k) { k.ln_eps = 0.0f; });
    bad_k([](dsaidx_k_args& k) { k.ln_eps = -1e-6f; });
    bad_k([](dsaidx_k_args& k) { k.ln_eps = NAN; });
    bad_k([](dsaidx_k_args& k) { k.ln_eps = INFINITY; });
    bad_k([](dsaidx_k_args& k) { k.flags = 0x8; });
    bad_k([](dsaidx_k_args& k) { k.flags = DSAIDX_K_BF16_INTERMEDIATE | DSAIDX_K_BF16_ROUND_ONCE; });
    bad_k([](dsaidx_k_args& k) { k.num_slots = 0; });
    bad_k([](dsaidx_k_args& k) { k.k_cache_row_stride = 120; });
    bad_k([](dsaidx_k_args& k) { k.k_cache_row_stride = 132; });
    bad_k([](dsaidx_k_args& k) {
        k.flags = DSAIDX_K_PAGED_CACHE;
        k.page_size = 96;  // does not divide num_slots = 4096
    });
    bad_k([](dsaidx_k_args& k) {
        k.flags = DSAIDX_K_PAGED_CACHE;
        k.page_size = 1;
    });
    bad_k([](dsaidx_k_args& k) {
        k.flags = DSAIDX_K_PAGED_CACHE;
        k.page_size = 3;
        k.num_slots = 3 * 1024;
    });
    CHECK(g_launches.empty());
}

void topk_and_selftest() {
    const float* lg = at<const float>(0);
    int32_t* out = at<int32_t>(32768);
    void* ws = at<void>(40960);
    g_launches.clear();
    CHECK(dsaidx_topk_per_row(lg, 1000, nullptr, 0, 1000, 10, out, nullptr, 0, nullptr) == DSAIDX_OK);
    CHECK(g_launches.empty());
    CHECK(dsaidx_topk_workspace_bytes(3, 1000, 10) == 0);
    CHECK(dsaidx_topk_workspace_bytes(3, 40000, 10) == 3 * (8224 + 8 * 4096));
    CHECK(dsaidx_topk_workspace_bytes(3, 40000, 0) == -1);
    CHECK(dsaidx_topk_workspace_bytes(-1, 40000, 10) == -1);
    CHECK(dsaidx_topk_per_row(lg, 1000, nullptr, 3, 1000, 10, out, nullptr, 0, nullptr) == DSAIDX_OK);
    CHECK(g_launches.size() == 1 && g_launches[0].kind == 1 && g_launches[0].rows == 3);
    const int64_t need = 3 * (8224 + 8 * 4096);
    CHECK(dsaidx_topk_per_row(lg, 40000, at<const int32_t>(1024), 3, 40000, 10, out, ws, need, nullptr) ==
          DSAIDX_OK);
    CHECK(g_launches.size() == 2 && g_launches[1].workspace == ws);
    REJECT(dsaidx_topk_per_row(lg, 40000, nullptr, 3, 40000, 10, out, nullptr, need, nullptr));
    REJECT(dsaidx_topk_per_row(lg, 40000, nullptr, 3, 40000, 10, out, at<void>(40968), need, nullptr));
    REJECT(dsaidx_topk_per_row(lg, 40000, nullptr, 3, 40000, 10, out, ws, need - 1, nullptr));
    REJECT(dsaidx_topk_per_row(lg, 1000, nullptr, 3, 1000, 0, out, nullptr, 0, nullptr));
    REJECT(dsaidx_topk_per_row(lg, 1000, nullptr, 3, 1000, (1 << 20) + 1, out, nullptr, 0, nullptr));
    REJECT(dsaidx_topk_per_row(lg, 1000, nullptr, -1, 1000, 10, out, nullptr, 0, nullptr));
    REJECT(dsaidx_topk_per_row(lg, 996, nullptr, 3, 1000, 10, out, nullptr, 0, nullptr));
    REJECT(dsaidx_topk_per_row(lg, 1002, nullptr, 3, 1000, 10, out, nullptr, 0, nullptr));
    REJECT(dsaidx_topk_per_row(at<const float>(4), 1000, nullptr, 3, 1000, 10, out, nullptr, 0, nullptr));
    REJECT(dsaidx_topk_per_row(lg, 1000, at<const int32_t>(1026), 3, 1000, 10, out, nullptr, 0, nullptr));
    REJECT(dsaidx_topk_per_row(lg, 1000, nullptr, 3, 1000, 10, nullptr, nullptr, 0, nullptr));
    REJECT(dsaidx_topk_per_row(nullptr, 1000, nullptr, 3, 1000, 10, out, nullptr, 0, nullptr));
    g_launches.clear();
    CHECK(dsaidx_fp8_encode_selftest(lg, at<uint8_t>(32768), 0, 0, nullptr) == DSAIDX_OK);
    CHECK(g_launches.empty());
    CHECK(dsaidx_fp8_encode_selftest(lg, at<uint8_t>(32768), 1000, -22, nullptr) == DSAIDX_OK);
    CHECK(g_launches.size() == 1 && g_launches[0].kind == 2 && g_launches[0].grid == 1);
    CHECK(dsaidx_fp8_encode_selftest(lg, at<uint8_t>(32768), 1000, -126, nullptr) == DSAIDX_OK);
    CHECK(dsaidx_fp8_encode_selftest(lg, at<uint8_t>(32768), 1000, 127, nullptr) == DSAIDX_OK);
    REJECT(dsaidx_fp8_encode_selftest(lg, at<uint8_t>(32768), -1, 0, nullptr));
    REJECT(dsaidx_fp8_encode_selftest(lg, at<uint8_t>(32772), 8, 0, nullptr));
    REJECT(dsaidx_fp8_encode_selftest(nullptr, at<uint8_t>(32768), 8, 0, nullptr));
    REJECT(dsaidx_fp8_encode_selftest(lg, at<uint8_t>(32768), 8, -127, nullptr));
    REJECT(dsaidx_fp8_encode_selftest(lg, at<uint8_t>(32768), 8, 128, nullptr));
    // allocation-free top-k: rows of up to 32768 logits need no workspace and
    // take the ordinary launch; a workspace beyond the library's array is
    // refused before anything is looked up or enqueued
    g_launches.clear();
    CHECK(dsaidx_topk_per_row_noalloc(lg, 1000, nullptr, 3, 1000, 10, out, nullptr) == DSAIDX_OK);
    CHECK(g_launches.size() == 1 && g_launches[0].kind == 1 && g_launches[0].workspace == nullptr);
    CHECK(dsaidx::g_scratch_lookups == 0);
    g_launches.clear();
    CHECK(dsaidx_topk_per_row_noalloc(lg, 1000, nullptr, 0, 131072, 10, out, nullptr) == DSAIDX_OK);
    CHECK(g_launches.empty());
    REJECT(dsaidx_topk_per_row_noalloc(lg, 131072, nullptr, 228, 131072, 2048, out, nullptr));
    REJECT(dsaidx_topk_per_row_noalloc(lg, 1000, nullptr, 3, 1000, 0, out, nullptr));
    CHECK(dsaidx::g_scratch_lookups == 0);
    // split rows: the library's array serves as the workspace
    g_launches.clear();
    CHECK(dsaidx_topk_per_row_noalloc(lg, 131072, nullptr, 227, 131072, 2048, out, nullptr) ==
          DSAIDX_OK);
    CHECK(g_launches.size() == 1 && g_launches[0].workspace == reinterpret_cast<void*>(uintptr_t(1) << 40));
    CHECK(dsaidx::g_scratch_lookups == 1);
    // a stream of another device than the current one is refused
    g_stream_device = 1;
    g_launches.clear();
    CHECK(dsaidx_topk_per_row_noalloc(lg, 131072, nullptr, 4, 131072, 2048, out,
                                      reinterpret_cast<dsaidx_stream_t>(uintptr_t(64))) ==
          DSAIDX_ERR_INVALID_ARGUMENT);
    CHECK(g_launches.empty());
    g_stream_device = 0;
    // reference HBM streams: byte count in 16-byte vectors, nothing for 0 bytes
    g_launches.clear();
    CHECK(dsaidx_hbm_stream(DSAIDX_HBM_COPY, lg, at<uint8_t>(32768), 0, 0, nullptr) == DSAIDX_OK);
    CHECK(g_launches.empty());
    CHECK(dsaidx_hbm_stream(DSAIDX_HBM_READ, lg, at<uint8_t>(32768), 4096, 7, nullptr) == DSAIDX_OK);
    CHECK(g_launches.size() == 1 && g_launches[0].kind == 4 && g_launches[0].n == 256 &&
          g_launches[0].style == DSAIDX_HBM_READ);
    REJECT(dsaidx_hbm_stream(DSAIDX_HBM_WRITE, nullptr, at<uint8_t>(32776), 64, 0, nullptr));
    REJECT(dsaidx_hbm_stream(DSAIDX_HBM_COPY, lg, at<uint8_t>(32768), 40, 0, nullptr));
    REJECT(dsaidx_hbm_stream(7, lg, at<uint8_t>(32768), 64, 0, nullptr));
}

}  // namespace

void logits_calls() {
    auto make = [](int64_t T, int32_t H, int64_t N) {
        dsaidx_logits_args a;
        std::memset(&a, 0, sizeof a);
        a.q_fp8 = at<const uint8_t>(0);
        a.weights = at<const float>(8192);
        a.num_tokens = T;
        a.num_heads = H;
        a.k_cache = at<const uint8_t>(16384);
        a.k_cache_row_stride = 128;
        a.k_scale = at<const float>(32768);
        a.num_slots = 1 << 20;
        a.num_keys = N;
        a.logits = at<float>(40960);
        a.logits_stride = N;
        return a;
    };
    g_launches.clear();
    // key chunks: enough workgroups (about 3072 of 8 tokens each), at least 256 keys, whole stages;
    // chunk-major workgroup order when there are at least as many token blocks as chunks
    {
        dsaidx_logits_args a = make(64, 64, 16384);
        CHECK(dsaidx_mqa_logits(&a, nullptr) == DSAIDX_OK);
        a = make(8192, 64, 8192);
        CHECK(dsaidx_mqa_logits(&a, nullptr) == DSAIDX_OK);
        a = make(5, 3, 100);
        a.key_slots = at<const int32_t>(48000);
        a.lengths = at<const int32_t>(49000);
        CHECK(dsaidx_mqa_logits(&a, nullptr) == DSAIDX_OK);
        CHECK(g_launches.size() == 3);
        CHECK(g_launches[0].kind == 3 && g_launches[0].lp.chunk == 256 && g_launches[0].lp.chunks == 64);
        CHECK(g_launches[0].lp.chunk_major == 0);
        CHECK(g_launches[1].lp.chunk == 2816 && g_launches[1].lp.chunks == 3);
        CHECK(g_launches[1].lp.chunk_major == 1);
        CHECK(g_launches[2].lp.chunk == 128 && g_launches[2].lp.chunks == 1);
        CHECK(g_launches[2].lp.H == 3 && g_launches[2].lp.N == 100 && g_launches[2].lp.page_size == 0);
        CHECK(g_launches[2].lp.key_slots != nullptr && g_launches[2].lp.lengths != nullptr);
        // the workgroup index splits by the magic-number division the kernel
        // uses: checked for every workgroup of each grid
        for (const auto& l : g_launches) {
            const uint32_t d = l.lp.chunk_major ? (uint32_t)l.lp.blocks : (uint32_t)l.lp.chunks;
            CHECK(l.lp.blocks == (l.lp.T + 7) / 8);
            // one token per wavefront: one resident round, and the workgroups'
            // 16 strided key blocks cover every key
            CHECK(l.lp.tokens_per_wave == ((int64_t)l.lp.blocks * l.lp.chunks <= 512 ? 1 : 2));
            if (l.lp.tokens_per_wave == 1) CHECK((int64_t)l.lp.chunks * 256 >= l.lp.N);
            for (uint32_t b = 0; b < (uint32_t)l.lp.blocks * (uint32_t)l.lp.chunks; ++b)
                CHECK((uint32_t)(((uint64_t)b * l.lp.grid_magic) >> l.lp.grid_shift) == b / d);
        }
    }
    // the same division at the largest grid index and awkward divisors
    {
        g_launches.clear();
        dsaidx_logits_args a = make((int64_t(1) << 31) - 8, 1, 1);   // 2^28 - 1 token blocks, one chunk
        a.logits_stride = 1;
        CHECK(dsaidx_mqa_logits(&a, nullptr) == DSAIDX_OK);
        a = make(8 * 3, 64, (int64_t(1) << 31) - 1);                   // 3 token blocks, many chunks
        a.num_slots = a.num_keys;
        CHECK(dsaidx_mqa_logits(&a, nullptr) == DSAIDX_OK);
        CHECK(g_launches.size() == 2);
        for (const auto& l : g_launches) {
            const uint32_t d = l.lp.chunk_major ? (uint32_t)l.lp.blocks : (uint32_t)l.lp.chunks;
            const uint32_t n = (uint32_t)l.lp.blocks * (uint32_t)l.lp.chunks;
            for (uint32_t b : {0u, 1u, d - 1, d, d + 1, n / 2, n - 2, n - 1})
                if (b < n) CHECK((uint32_t)(((uint64_t)b * l.lp.grid_magic) >> l.lp.grid_shift) == b / d);
        }
    }
    // page-interleaved cache; empty calls
    {
        g_launches.clear();
        dsaidx_logits_args a = make(4, 64, 300);
        a.flags = DSAIDX_K_PAGED_CACHE;
        a.page_size = 64;
        a.k_scale = nullptr;
        a.k_cache_row_stride = 0;
        a.num_slots = 4096;
        CHECK(dsaidx_mqa_logits(&a, nullptr) == DSAIDX_OK);
        CHECK(g_launches.size() == 1 && g_launches[0].lp.page_size == 64 && g_launches[0].lp.k_scale == nullptr);
        a = make(0, 64, 300);
        a.q_fp8 = nullptr;
        CHECK(dsaidx_mqa_logits(&a, nullptr) == DSAIDX_OK);
        a = make(4, 64, 0);
        CHECK(dsaidx_mqa_logits(&a, nullptr) == DSAIDX_OK);
        CHECK(g_launches.size() == 1);
    }
    auto bad = [&](void (*edit)(dsaidx_logits_args&)) {
        dsaidx_logits_args a = make(16, 64, 1000);
        edit(a);
        REJECT(dsaidx_mqa_logits(&a, nullptr));
    };
    REJECT(dsaidx_mqa_logits(nullptr, nullptr));
    bad([](dsaidx_logits_args& a) { a.num_tokens = -1; });
    bad([](dsaidx_logits_args& a) { a.num_tokens = int64_t(1) << 31; });
    bad([](dsaidx_logits_args& a) { a.num_keys = -1; });
    bad([](dsaidx_logits_args& a) { a.num_keys = int64_t(1) << 31; a.logits_stride = a.num_keys; });
    bad([](dsaidx_logits_args& a) { a.num_heads = 0; });
    bad([](dsaidx_logits_args& a) { a.num_heads = 65; });
    bad([](dsaidx_logits_args& a) { a.q_fp8 = nullptr; });
    bad([](dsaidx_logits_args& a) { a.weights = nullptr; });
    bad([](dsaidx_logits_args& a) { a.k_cache = nullptr; });
    bad([](dsaidx_logits_args& a) { a.logits = nullptr; });
    bad([](dsaidx_logits_args& a) { a.q_fp8 = at<const uint8_t>(8); });          // 8-byte aligned only
    bad([](dsaidx_logits_args& a) { a.weights = at<const float>(8194); });
    bad([](dsaidx_logits_args& a) { a.k_cache = at<const uint8_t>(16388); });
    bad([](dsaidx_logits_args& a) { a.logits = at<float>(40962); });
    bad([](dsaidx_logits_args& a) { a.key_slots = at<const int32_t>(48002); });
    bad([](dsaidx_logits_args& a) { a.lengths = at<const int32_t>(49001); });
    bad([](dsaidx_logits_args& a) { a.flags = DSAIDX_K_BF16_INTERMEDIATE; });
    bad([](dsaidx_logits_args& a) { a.num_slots = 0; });
    bad([](dsaidx_logits_args& a) { a.num_slots = 999; });                      // fewer slots than keys
    bad([](dsaidx_logits_args& a) { a.logits_stride = 999; });
    bad([](dsaidx_logits_args& a) { a.k_scale = nullptr; });
    bad([](dsaidx_logits_args& a) { a.k_cache_row_stride = 120; });
    bad([](dsaidx_logits_args& a) { a.k_cache_row_stride = 132; });
    bad([](dsaidx_logits_args& a) {
        a.flags = DSAIDX_K_PAGED_CACHE;
        a.page_size = 96;                                                         // does not divide 2^20
    });
    bad([](dsaidx_logits_args& a) {
        a.flags = DSAIDX_K_PAGED_CACHE;
        a.page_size = 3;
        a.num_slots = 3 << 10;
    });
}

// The projection entry: one dispatch of ceil(T / kProjRows) workgroups, the key
// side filled as for the key entry (its row pointer unused), every rejected
// argument enqueuing nothing.
void projection_calls() {
    dsaidx_rope rope = make_rope();
    auto proj = [](int64_t d, int32_t H) {
        dsaidx_proj_args j;
        std::memset(&j, 0, sizeof j);
        j.hidden = at<const uint16_t>(1 << 20);
        j.hidden_stride_t = d;
        j.weight = at<const uint16_t>(1 << 22);
        j.weight_stride_n = d;
        j.hidden_dim = d;
        j.num_heads = H;
        j.gates_out = at<uint16_t>(1 << 24);
        j.gates_stride_t = H;
        return j;
    };
    dsaidx_k_args k = make_k(300);
    k.k = nullptr;
    k.k_stride_t = 0;
    g_launches.clear();
    dsaidx_proj_args j = proj(7168, 64);
    CHECK(dsaidx_proj_k_norm_rope_quant_store(&j, &k, &rope, nullptr) == DSAIDX_OK);
    CHECK(g_launches.size() == 1 && g_launches[0].kind == 5);
    {   // the largest row strides accepted
        dsaidx_proj_args jw = proj(7168, 64);
        jw.hidden_stride_t = int64_t(1) << 22;
        jw.weight_stride_n = int64_t(1) << 22;
        CHECK(dsaidx_proj_k_norm_rope_quant_store(&jw, &k, &rope, nullptr) == DSAIDX_OK);
        g_launches.clear();
        CHECK(dsaidx_proj_k_norm_rope_quant_store(&j, &k, &rope, nullptr) == DSAIDX_OK);
    }
    if (!g_launches.empty()) {
        const Launch& l = g_launches[0];
        const int64_t blocks = (300 + dsaidx::kProjRows - 1) / dsaidx::kProjRows;
        CHECK(l.grid == blocks && l.rows == blocks && l.n == 7168 && l.k == 64 && l.style == 0);
        CHECK(l.p.T == 300 && l.p.k == nullptr && l.p.loc == k.out_cache_loc && l.p.S == k.num_slots);
        CHECK(l.workspace == nullptr);
    }
    // T = 0: nothing, whatever the pointers
    g_launches.clear();
    dsaidx_k_args k0 = make_k(0);
    dsaidx_proj_args j0;
    std::memset(&j0, 0, sizeof j0);
    CHECK(dsaidx_proj_k_norm_rope_quant_store(&j0, &k0, &rope, nullptr) == DSAIDX_OK);
    CHECK(g_launches.empty());
    auto bad = [&](void (*edit)(dsaidx_proj_args&, dsaidx_k_args&)) {
        dsaidx_proj_args jj = proj(7168, 64);
        dsaidx_k_args kk = k;
        edit(jj, kk);
        REJECT(dsaidx_proj_k_norm_rope_quant_store(&jj, &kk, &rope, nullptr));
    };
    bad([](dsaidx_proj_args& j, dsaidx_k_args&) { j.hidden_dim = 96; });
    bad([](dsaidx_proj_args& j, dsaidx_k_args&) { j.hidden_dim = 0; });
    bad([](dsaidx_proj_args& j, dsaidx_k_args&) { j.num_heads = 65; });
    bad([](dsaidx_proj_args& j, dsaidx_k_args&) { j.hidden = nullptr; });
    bad([](dsaidx_proj_args& j, dsaidx_k_args&) { j.weight_stride_n = 7000; });
    bad([](dsaidx_proj_args& j, dsaidx_k_args&) { j.hidden_stride_t = (int64_t(1) << 22) + 8; });
    bad([](dsaidx_proj_args& j, dsaidx_k_args&) { j.weight_stride_n = (int64_t(1) << 22) + 8; });
    bad([](dsaidx_proj_args& j, dsaidx_k_args&) { j.gates_stride_t = 32; });
    bad([](dsaidx_proj_args& j, dsaidx_k_args&) { j.k_out = at<uint16_t>(8); j.k_out_stride_t = 128; });
    bad([](dsaidx_proj_args&, dsaidx_k_args& k) { k.ln_eps = 0.0f; });
    bad([](dsaidx_proj_args&, dsaidx_k_args& k) { k.k_cache = nullptr; });
    CHECK(dsaidx_proj_k_norm_rope_quant_store(nullptr, &k, &rope, nullptr) == DSAIDX_ERR_INVALID_ARGUMENT);
}

int main() {
    abi_and_status();
    projection_calls();
    logits_calls();
    launch_shapes();
    rejected_arguments();
    topk_and_selftest();
    if (g_errors) {
        std::fprintf(stderr, "%d check(s) failed\n", g_errors);
        return 1;
    }
    std::printf("host layer: all checks passed\n");
    return 0;
}
