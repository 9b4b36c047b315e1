"""MI355X-native top-k / top-p logits filter (libtopktopp) and its Python binding."""

from .binding import (  # noqa: F401
    EXPORTED_SYMBOLS,
    LIB_PATH,
    TopKTopPError,
    apply_top_k_top_p,
    apply_top_k_top_p_with_sorted,
    last_error,
    load_library,
    sample_top_k_top_p,
    set_plan_policy,
    top_k_top_p_sorted_survivors,
)
