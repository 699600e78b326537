// Test double of the kernel launchers for the host sanitizer build of the C
// ABI front end (tests/test_sanitizers.py): the front end's validation runs
// for real, the launches only check the parameter block they receive and
// count.  The HIP device queries the allocation-free entry point makes are
// answered for device 0.
#include "../../gateddeltanet_chunked_delta_amd/csrc/gdn_internal.h"
#include "../../include/gdn.h"

#include <stdio.h>
#include <stdlib.h>

namespace gdn {

static int g_launches = 0;

static void expect(bool ok, const char* what) {
    if (!ok) {
        fprintf(stderr, "stub launcher: %s\n", what);
        abort();
    }
}

hipError_t launch_prefill(const PrefillParams& p, int d_k, int d_v, int qkv_dtype, int out_dtype, hipStream_t,
                          void* const*) {
    expect(p.num_seqs > 0 && p.h_k > 0 && p.h_v % p.h_k == 0 && p.d_v == d_v, "prefill sizes");
    expect(prefill_supported(d_k, d_v, qkv_dtype, out_dtype) != 0, "prefill kernel choice");
    expect(p.q && p.k && p.v && p.g && p.beta && p.o && p.cu_seqlens, "prefill pointers");
    expect(p.order && p.chunk_base && p.slot_desc && p.kq_img && p.tp_img && p.scal_img, "workspace regions");
    expect((reinterpret_cast<uintptr_t>(p.kq_img) & 255) == 0 && (reinterpret_cast<uintptr_t>(p.tp_img) & 255) == 0,
           "workspace alignment");
    expect(p.segment_chunks == 0 ? !p.chain_base && !p.seg_y
                                 : p.chain_base && p.chain_desc && p.chain_order && p.seg_state && p.seg_trans &&
                                       p.seg_y && p.seg_oloc && p.max_chains >= p.num_seqs,
           "segment split buffers");
    g_launches++;
    return hipSuccess;
}

hipError_t launch_decode(const DecodeParams& p, int d_k, int d_v, int qkv_dtype, int out_dtype, hipStream_t) {
    expect(p.num_seqs > 0 && p.tokens >= 1 && p.tokens <= kDecodeMaxTokens, "decode sizes");
    expect(decode_supported(d_k, d_v, qkv_dtype, out_dtype) != 0, "decode kernel choice");
    expect(p.q && p.k && p.v && p.g && p.beta && p.o && p.state_pool, "decode pointers");
    g_launches++;
    return hipSuccess;
}

hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
    *ptr = reinterpret_cast<void*>(uintptr_t(0x7f0000000000ull));  // a 256-byte aligned stand-in, never dereferenced
    *bytes = GDN_NOALLOC_SCRATCH_BYTES;
    return hipSuccess;
}

}  // namespace gdn

extern "C" {
hipError_t hipGetDevice(int* device) {
    *device = 0;
    return hipSuccess;
}
hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t* device) {
    *device = 0;
    return hipSuccess;
}
int gdn_stub_launches(void) { return gdn::g_launches; }
}

namespace gdn {
hipError_t launch_stream_copy(void*, const void*, int64_t, int, hipStream_t) {
    g_launches++;
    return hipSuccess;
}
}  // namespace gdn
