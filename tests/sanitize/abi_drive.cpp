// Drives the host side of every librtp entry point -- argument checks, error
// text, workspace sizing -- with valid and invalid arguments, for the
// AddressSanitizer / UndefinedBehaviorSanitizer build of the library's host
// code.  No call here reaches a kernel launch, so no GPU is needed.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/rtp.h"

#define CHECK(c)                                                                   \
    do {                                                                           \
        if (!(c)) {                                                                \
            std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__);    \
            return 1;                                                              \
        }                                                                          \
    } while (0)

static void* const FAKE = reinterpret_cast<void*>(0x1000);

int main() {
    rtp_layer L;
    std::memset(&L, 0, sizeof L);
    L.num_q_heads = 32;
    L.num_kv_heads = 8;
    L.head_dim = 128;
    L.dtype = RTP_BF16;
    L.num_ret = 3;
    L.ret_heads[0] = 1;
    L.ret_heads[1] = 5;
    L.ret_heads[2] = 9;
    L.window = 2048;
    L.num_sinks = 64;
    L.attn_scale = 0.088f;
    L.idx_scale = 0.25f;
    rtp_cache C;
    std::memset(&C, 0, sizeof C);
    C.k = C.v = FAKE;
    C.k_low = FAKE;
    C.block_table = C.seq_lens = static_cast<const int32_t*>(FAKE);
    C.batch = 2;
    C.max_blocks = 4096;
    C.max_seq_len = 1 << 20;
    rtp_query Q;
    std::memset(&Q, 0, sizeof Q);
    Q.q = FAKE;
    Q.n_tok = 2;
    Q.kind = RTP_DECODE;
    rtp_sel S;
    S.row_ptr = static_cast<int64_t*>(FAKE);
    S.idx = static_cast<int32_t*>(FAKE);
    S.status = static_cast<int32_t*>(FAKE);
    S.capacity = 100;

    CHECK(rtp_version() == RTP_VERSION);
    const size_t ws = rtp_topp_select_workspace(&L, &C, &Q);
    CHECK(ws > 0 && rtp_topp_select_workspace_min(&L, &C, &Q) == ws);
    CHECK(rtp_sparse_attn_workspace(&L, &C, &Q, 1000) > 0);
    CHECK(rtp_window_attn_workspace(&L, &C, &Q) > 0 && rtp_dense_attn_workspace(&L, &C, &Q) > 0);
    rtp_query P = Q;
    P.kind = RTP_CHUNK;
    P.n_tok = 8192;
    P.pos0 = (1 << 20) - 8192;
    C.batch = 1;
    CHECK(rtp_topp_select_workspace(&L, &C, &P) > rtp_topp_select_workspace_min(&L, &C, &P));
    CHECK(rtp_sparse_attn_workspace(&L, &C, &P, 1 << 20) > 0);
    C.batch = 2;
    // workspace too small: rejected before any launch
    CHECK(rtp_topp_select(&L, &C, &Q, FAKE, static_cast<const float*>(FAKE), &S, FAKE, ws - 1, nullptr) ==
          RTP_EWORKSPACE);
    CHECK(std::strlen(rtp_last_error()) > 0);
    {
        rtp_cache W = C;                                  // 48 decode rows over 2^20 keys: beyond the static scratch
        W.batch = 16;
        rtp_query WQ = Q;
        WQ.n_tok = 16;
        CHECK(rtp_topp_select_noalloc(&L, &W, &WQ, FAKE, static_cast<const float*>(FAKE), &S, nullptr) ==
              RTP_EWORKSPACE);
    }
    // invalid layers
    rtp_layer B = L;
    B.num_kv_heads = 7;
    CHECK(rtp_window_attn(&B, &C, &Q, FAKE, FAKE, 1u << 30, nullptr) == RTP_EINVAL);
    B = L;
    B.head_dim = 96;
    CHECK(rtp_window_attn(&B, &C, &Q, FAKE, FAKE, 1u << 30, nullptr) == RTP_EUNSUPPORTED);
    B = L;
    B.ret_heads[1] = 1;
    CHECK(rtp_indexer_append(&B, &C, FAKE, static_cast<const int32_t*>(FAKE), static_cast<const int32_t*>(FAKE), 4,
                             nullptr) == RTP_EINVAL);
    B = L;
    B.idx_scale = NAN;
    CHECK(rtp_topk_select(&B, &C, &Q, FAKE, 8, &S, FAKE, ws, nullptr) == RTP_EINVAL);
    B = L;
    B.kv_fp8 = 1;
    B.k_scale = 0.0f;
    B.v_scale = 1.0f;
    CHECK(rtp_kv_append(&B, &C, FAKE, FAKE, FAKE, static_cast<const int32_t*>(FAKE),
                        static_cast<const int32_t*>(FAKE), 4, nullptr) == RTP_EINVAL);
    B = L;
    B.flags = 8;
    CHECK(rtp_sparse_attn_decode(&B, &C, &Q, &S, FAKE, FAKE, 1u << 30, nullptr) == RTP_EINVAL);
    // invalid caches and queries
    rtp_cache D = C;
    D.max_seq_len = (1 << 20) + 1;
    CHECK(rtp_dense_attn(&L, &D, &Q, FAKE, FAKE, 1u << 30, nullptr) == RTP_EUNSUPPORTED);
    D = C;
    D.k_ring = FAKE;
    D.ring_pages = 1;
    CHECK(rtp_window_attn(&L, &D, &Q, FAKE, FAKE, 1u << 30, nullptr) == RTP_EINVAL);
    rtp_query E = Q;
    E.n_tok = 3;
    CHECK(rtp_sparse_attn_decode(&L, &C, &E, &S, FAKE, FAKE, 1u << 30, nullptr) == RTP_EINVAL);
    E = Q;
    E.kind = 9;
    CHECK(rtp_indexer_scores(&L, &C, &E, FAKE, static_cast<uint16_t*>(FAKE), static_cast<float*>(FAKE), 1 << 20,
                             nullptr) == RTP_EINVAL);
    CHECK(rtp_sparse_attn_prefill(&L, &C, &Q, &S, FAKE, FAKE, 1u << 30, nullptr) == RTP_EINVAL);
    CHECK(rtp_topp_select_paths(&L, &C, &Q, FAKE, ws, nullptr, nullptr) == RTP_EINVAL);
    CHECK(rtp_topk_select(&L, &C, &Q, FAKE, 0, &S, FAKE, ws, nullptr) == RTP_EINVAL);
    CHECK(rtp_indexer_append(&L, &C, FAKE, static_cast<const int32_t*>(FAKE), static_cast<const int32_t*>(FAKE), 0,
                             nullptr) == RTP_OK);
    CHECK(rtp_kv_append(&L, &C, FAKE, FAKE, FAKE, static_cast<const int32_t*>(FAKE),
                        static_cast<const int32_t*>(FAKE), -1, nullptr) == RTP_EINVAL);
    std::printf("abi drive ok\n");
    return 0;
}
