// Output stores of the stand-alone streaming kernels (dequantisation, merge):
// written once and not read again by the kernel, so they carry the
// non-temporal hint and do not displace cached inputs.
#pragma once

namespace lora {

template <typename V>
__device__ __forceinline__ void store_stream(V* p, const V& v) {
#ifdef LORA_NO_NT_STORE
    *p = v;
#else
    __builtin_nontemporal_store(v, p);
#endif
}

}  // namespace lora
