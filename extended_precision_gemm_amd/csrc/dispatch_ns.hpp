// Run-time slice count -> compile-time template argument, host side.
#pragma once

#include <type_traits>

namespace ddg {

// Calls fn(std::integral_constant<int, NS>) for a run-time slice count 4..16.
template <class Fn>
auto dispatch_ns(int ns, Fn&& fn) -> decltype(fn(std::integral_constant<int, 8>{})) {
    switch (ns) {
        case 4: return fn(std::integral_constant<int, 4>{});
        case 5: return fn(std::integral_constant<int, 5>{});
        case 6: return fn(std::integral_constant<int, 6>{});
        case 7: return fn(std::integral_constant<int, 7>{});
        case 8: return fn(std::integral_constant<int, 8>{});
        case 9: return fn(std::integral_constant<int, 9>{});
        case 10: return fn(std::integral_constant<int, 10>{});
        case 11: return fn(std::integral_constant<int, 11>{});
        case 12: return fn(std::integral_constant<int, 12>{});
        case 13: return fn(std::integral_constant<int, 13>{});
        case 14: return fn(std::integral_constant<int, 14>{});
        case 15: return fn(std::integral_constant<int, 15>{});
        case 16: return fn(std::integral_constant<int, 16>{});
        default: return decltype(fn(std::integral_constant<int, 8>{}))();
    }
}

}  // namespace ddg
