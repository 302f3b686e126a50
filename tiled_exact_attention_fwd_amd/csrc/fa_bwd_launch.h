// Launchers of the backward kernel instances (one translation unit per
// element type and head dimension); each returns 0, or -1 if a launch failed.
// `cus` is the device's compute-unit count (it sizes the causal block order).
#pragma once

namespace fa {
namespace bwd {

struct BwdParams;
struct BwdParams32;

int launch_bwd_bf16_d64(const BwdParams& p, int heads, int cus, bool causal, void* stream);
int launch_bwd_bf16_d128(const BwdParams& p, int heads, int cus, bool causal, void* stream);
int launch_bwd_f16_d64(const BwdParams& p, int heads, int cus, bool causal, void* stream);
int launch_bwd_f16_d128(const BwdParams& p, int heads, int cus, bool causal, void* stream);
// fp32, d = 64 or 128
int launch_bwd_f32(const BwdParams32& p, int heads, int d, bool causal, void* stream);

}  // namespace bwd
}  // namespace fa
