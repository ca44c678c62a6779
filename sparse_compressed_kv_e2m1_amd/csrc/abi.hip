// abi.hip -- error reporting and workspace sizing shared by the C ABI calls.
#include <string>

#include "sckv_device.h"

namespace sckv {

size_t index_workspace_bytes(int B, int64_t m, int64_t n_c);
size_t index_fp4_workspace_bytes(int B, int64_t m, int64_t n_c);
size_t attn_workspace_bytes(int B, int64_t m, int H, int D, int64_t T);

namespace {
thread_local std::string g_last_error;
}

void set_error(const std::string& msg) { g_last_error = msg; }

int fail(int code, const std::string& msg) {
    set_error(msg);
    return code;
}

int check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SCKV_EHIP, std::string(what) + ": " + hipGetErrorString(e));
    return SCKV_OK;
}

}  // namespace sckv

extern "C" size_t sckv_workspace_bytes(int op, int B, int64_t m, int H, int D, int64_t n) {
    if (B < 0 || m < 0 || H <= 0 || D <= 0 || n < 0) return (size_t)-1;
    if (op == SCKV_OP_INDEX_SCORES_TOPK) return sckv::index_workspace_bytes(B, m, n);
    if (op == SCKV_OP_SPARSE_ATTN_SINK) return sckv::attn_workspace_bytes(B, m, H, D, n);
    if (op == SCKV_OP_INDEX_SCORES_TOPK_FP4) return sckv::index_fp4_workspace_bytes(B, m, n);
    return (size_t)-1;
}

extern "C" const char* sckv_last_error(void) { return sckv::g_last_error.c_str(); }

extern "C" int sckv_abi_version(void) { return 2; }
